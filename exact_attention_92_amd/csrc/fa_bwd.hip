// The fa_bwd entry point declared in include/fa_api.h and the head-dimension
// 128 instantiation of the backward kernels (fa_bwd_kernels.h describes the
// method and the kernels; fa_bwd_d64.hip holds the d = 64 instantiation).
#include "fa_bwd_kernels.h"

namespace {

int check_bwd_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, const void* dq, const void* dk, const void* dv,
                   const float* dps, int B, int H, int N, int d, float scale, int mask_kind,
                   const int32_t* kv_lens) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !dps)
    return FA_ERR_INVALID_ARG;
  const uintptr_t al = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o |
                       (uintptr_t)lse | (uintptr_t)dout | (uintptr_t)dq | (uintptr_t)dk |
                       (uintptr_t)dv | (uintptr_t)dps;
  if (al & 15u) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
  if (mask_kind & ~(FA_MASK_CAUSAL | FA_MASK_KEY_PADDING)) return FA_ERR_INVALID_ARG;
  if ((mask_kind & FA_MASK_KEY_PADDING) && !kv_lens) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const long long nb = ((long long)N + 127) / 128;
  if ((long long)B * H * nb > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  // One head's rows (plus one block past the end) use 32-bit byte offsets.
  if (((long long)N + 256) * d * 4 > 0xffffffffLL) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

}  // namespace

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      float* dp_rowsum, int B, int H, int N, int d, float scale, int mask_kind,
                      const int32_t* kv_lens, void* stream) {
  const int st = check_bwd_args(q, k, v, o, lse, dout, dq, dk, dv, dp_rowsum, B, H, N, d, scale,
                                mask_kind, kv_lens);
  if (st != FA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dps = dp_rowsum;
  p.kv_lens = (mask_kind & FA_MASK_KEY_PADDING) ? kv_lens : nullptr;
  p.H = H;
  p.N = N;
  float a = fabsf(scale);
  if (a < kMinScale) a = kMinScale;
  p.c = a * kLog2e;
  p.gscale = (signbit(scale) && scale != 0.f) ? -a : a;
  p.ascale = a;
  p.qsign = (signbit(scale) && scale != 0.f) ? 0x80008000u : 0u;
  p.causal = (mask_kind & FA_MASK_CAUSAL) ? 1 : 0;

  // The second kernel reads the D written by the first: both go on s, in order.
  const bool ok = d == 128 ? launch_bwd<128>(p, B, s) : bwd_launch_d64(p, B, s);
  return ok ? FA_OK : FA_ERR_HIP;
}
