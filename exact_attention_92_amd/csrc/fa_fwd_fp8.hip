// FP8 (E4M3) attention forward for gfx950 (MI355X) and the fa_fwd_fp8 entry
// point declared in include/fa_api.h.
//
// Same computation as the bf16 forward (the online softmax of "FlashAttention
// 算法详解：从IO瓶颈到Triton实现", sections Online Softmax and FlashAttention
// Forward流程), on the FP8 path that §5.5 of "FlashAttention 完整解析"
// (freezetheflame.cc) and §9.2 of the youngju.dev walkthrough describe: Q, K
// and V arrive as E4M3 values with scale factors, the products run on the
// FP8 matrix cores with a wider accumulator, and the probabilities are scaled
// per tile before they are rounded to FP8, so that they do not underflow.
//
// Mapping to CDNA4:
//
//  * v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands, neutral block scales):
//    twice the bf16 rate, fp32 accumulation.  Key blocks are 128 keys long
//    at d = 128 (the softmax work dominates, so the per-block loop, barrier
//    and staging work is spread over more keys), 64 at d = 64; each 64-key
//    part is one 64-deep P V step.
//  * As in the bf16 kernel, scores are computed transposed (S^T = K Q^T, one
//    query row per lane) with the K rows permuted so the registers of a lane
//    hold 32 keys in a fixed order; V^T is stored in LDS with its keys in
//    that same order, so the rounded probabilities are directly the B
//    operand of O^T = V^T P^T (two 16-byte LDS reads per operand).
//  * The reference for the exponentials is the row max, moved only when a
//    block's max exceeds it by more than kHeadroom (log2 units), so every
//    probability is at most 2^kHeadroom and most blocks skip the rescaling of
//    the state (any reference gives the same softmax).  P is scaled by
//    448 / 2^kHeadroom (448 is the largest E4M3 value) before rounding --
//    folded into the exponent -- which keeps values down to ~2e-5
//    representable.  The factor and the V scale are divided out once in the
//    epilogue; the row sum is the fp32 sum of the unrounded scaled
//    probabilities (it also gives LSE).
//  * The per-head Q and K scales fold into the exp2 constant, the V scale
//    into the final division.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_api.h"
#include "fa_device.h"

namespace {

using namespace fa92;

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// log2(448); 448 is the largest finite E4M3 value.
constexpr float kLog2P8Scale = 8.807354922057604f;
// Probabilities may exceed 1 by up to 2^kHeadroom before the reference moves.
#ifndef FA_FP8_HEADROOM
#define FA_FP8_HEADROOM 2
#endif
constexpr float kHeadroom = (float)FA_FP8_HEADROOM;
constexpr float kLog2PScale = kLog2P8Scale - kHeadroom;   // log2(448 / 2^kHeadroom)

// D = A B + C, 32x32 tile, 64-deep E4M3 contraction, fp32 accumulation.
// Lane l supplies A row / B column l%32, 32 contraction elements per lane
// half; C as in the bf16 MFMA.  Block scales 127 are 2^0 (no scaling).
__device__ __forceinline__ f32x16_t mfma_fp8(i32x8_t a, i32x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8_t join(u32x4_t lo, u32x4_t hi) {
  return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Four floats (already scaled into [0, 448]) -> four E4M3 bytes, nearest even.
__device__ __forceinline__ unsigned pack_fp8x4(float a, float b, float c, float d) {
  // The first conversion writes the low half-word; the second the high one
  // (the old-value operand of the first is never seen, so any register
  // already holding a value does, without a move).
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (unsigned)w;
}

// Position of key k (0..127) of a block in the V^T tile.  Each 64-key half
// of the block is one 64-deep P V step; within it, lane half h of the P^T
// operand holds, in order, keys 16a + 8h + b of key tile t (a = 0..1,
// b = 0..7, t = 0..1) -- the score registers of the permuted S^T tiles.
__device__ __forceinline__ int vt_pos(int k) {
  return (k >> 6) * 64 + ((k >> 3) & 1) * 32 + ((k >> 5) & 1) * 16 + ((k >> 4) & 1) * 8 +
         (k & 7);
}

struct P8Params {
  const void* q;
  const void* k;
  const void* v;
  const float* q_descale;
  const float* k_descale;
  const float* v_descale;
  void* o;
  float* lse;
  const int32_t* kv_lens;
  int H, N, nqb;
  float ascale;     // |scale|, at least 1e-30
  unsigned qsign;   // E4M3 sign flip applied to Q when scale < 0
  int causal;
  int hg;           // heads map_work visits together (head_group)
  int nqt;          // per-tile scales: FA_FP8_TILE-row tiles per head (ceil(N / 128))
};

// TILED: q_descale and k_descale hold one scale per FA_FP8_TILE rows of each
// head (block quantization at tile granularity); a wave's 32 query rows lie
// in one Q tile and a key block in one K tile, so the scales enter the logit
// multiplier c per key block -- one scalar product per block.
template <int D, int NW, bool TILED>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
void fa_fwd_fp8_kernel(P8Params p) {
  constexpr int kThreads = 64 * NW;
  // Keys per block: 128 at d = 128 (two 64-deep P V steps; +16% over 64),
  // 64 at d = 64 (there 128 measured 10% slower).
  constexpr int BN = D >= 128 ? 128 : 64;
  constexpr int BM = 32 * NW;        // query rows per workgroup
  constexpr int NSB = BN / 64;       // 64-key halves of a block
  constexpr int KS = D / 64;         // 64-deep steps over d
  constexpr int DT = D / 32;         // 32-row tiles of O^T
  constexpr int KT = BN / 32;        // 32-key tiles of S^T
  constexpr int KLD = D + 16;        // K row stride in LDS (bytes)
  constexpr int VLD = BN + 16;       // V^T row stride in LDS (bytes)
  constexpr uint32_t ROWB = D;       // bytes per row in device memory
  constexpr int KP = BN * (D / 16);  // 16-byte K pieces per block
  constexpr int KU = (KP + kThreads - 1) / kThreads;
  constexpr int VUNITS = (BN / 4) * (D / 16);   // V pieces of 4 keys x 16 dims
  static_assert((KP % kThreads == 0 || KP < kThreads) && VUNITS <= kThreads, "tile shape");

  __shared__ __attribute__((aligned(16))) uint8_t k_lds[2][BN][KLD];
  __shared__ __attribute__((aligned(16))) uint8_t vt_lds[2][D][VLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const bool causal = p.causal != 0;
  const int N = p.N;

  int bh, qb;
  map_work(p.nqb, causal, p.hg, bh, qb);
  const int b = bh / p.H;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const uint8_t* Kh = (const uint8_t*)p.k + hoff;
  const uint8_t* Vh = (const uint8_t*)p.v + hoff;
  int n_vis = N;
  if (p.kv_lens) {
    const int kl = p.kv_lens[b];
    n_vis = kl < 0 ? 0 : (kl > N ? N : kl);
  }
  const int q0 = qb * BM;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + n;
  const int kend = causal ? min(n_vis, q0 + BM) : n_vis;
  const int nblk = (kend + BN - 1) / BN;

  // Logits in log2 units: s * |scale| * q_descale * k_descale * log2(e).
  static_assert(!TILED || BN <= FA_FP8_TILE, "a key block must lie in one scale tile");
  const float cq = p.ascale * (TILED ? p.q_descale[(size_t)bh * p.nqt + min(qw0 / FA_FP8_TILE,
                                                                             p.nqt - 1)]
                                     : p.q_descale[bh]);
  float c = fmaxf(cq * p.k_descale[bh], kMinScale) * kLog2e;

  // Q row of this lane: the B operand of S^T = K Q^T, bytes 64ks + 32hf + 0..31.
  i32x8_t qr[KS];
  {
    const rsrc_t rq = make_rsrc((const uint8_t*)p.q + hoff, (uint32_t)N * ROWB);
    const uint32_t off = (uint32_t)qrow * ROWB + 32u * hf;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qr[ks] = join(buf_load16(rq, off + 64u * ks) ^ p.qsign,
                    buf_load16(rq, off + 64u * ks + 16u) ^ p.qsign);
  }

  // Staging of key block j.  K: row-major 16-byte pieces.  V: pieces of 4
  // keys x 16 dims, byte-transposed into V^T rows at the permuted key
  // positions.  Buffer ranges end at N (K) and at the last visible key (V).
  uint32_t k_off[KU];
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int unit = tid + u * kThreads;
    k_off[u] = (uint32_t)(unit / (D / 16)) * ROWB + 16u * (unit % (D / 16));
  }
  const bool v_unit = tid < VUNITS;
  const int vkg = tid % (BN / 4), vdc = tid / (BN / 4);
  const uint32_t v_off = (uint32_t)(4 * vkg) * ROWB + 16u * vdc;
  const int v_col = vt_pos(4 * vkg);
  u32x4_t kreg[KU], vreg[4];
  auto load_block = [&](int j) {
    const int kbase = j * BN;
    const rsrc_t rk = make_rsrc(Kh + (size_t)kbase * D, (uint32_t)max(0, N - kbase) * ROWB);
    const rsrc_t rv = make_rsrc(Vh + (size_t)kbase * D, (uint32_t)max(0, n_vis - kbase) * ROWB);
#pragma unroll
    for (int u = 0; u < KU; ++u)
      if (KP >= kThreads || tid < KP) kreg[u] = buf_load16(rk, k_off[u]);
    if (v_unit) {
#pragma unroll
      for (int i = 0; i < 4; ++i) vreg[i] = buf_load16(rv, v_off + i * ROWB);
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int unit = tid + u * kThreads;
      if (KP >= kThreads || unit < KP)
        *(u32x4_t*)&k_lds[buf][unit / (D / 16)][16 * (unit % (D / 16))] = kreg[u];
    }
    if (v_unit) {
      // Dword w of key i holds dims 16vdc + 4w + 0..3: regroup the 4 keys'
      // bytes per dim (two rounds of v_perm_b32).
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const unsigned r0 = vreg[0][w], r1 = vreg[1][w], r2 = vreg[2][w], r3 = vreg[3][w];
        const unsigned t01l = __builtin_amdgcn_perm(r1, r0, 0x05010400u);
        const unsigned t01h = __builtin_amdgcn_perm(r1, r0, 0x07030602u);
        const unsigned t23l = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
        const unsigned t23h = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
        const int d0 = 16 * vdc + 4 * w;
        *(unsigned*)&vt_lds[buf][d0 + 0][v_col] = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u);
        *(unsigned*)&vt_lds[buf][d0 + 1][v_col] = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u);
        *(unsigned*)&vt_lds[buf][d0 + 2][v_col] = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u);
        *(unsigned*)&vt_lds[buf][d0 + 3][v_col] = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u);
      }
    }
  };

  float m_run = -INFINITY;   // running row max, log2 units (one query row per lane)
  float l_run = 0.f;         // running fp32 row sum
  f32x16_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();
  const int krow = row_perm(n);

  if (nblk > 0) {
    load_block(0);
    store_block(0);
  }
  __syncthreads();

  for (int j = 0; j < nblk; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < nblk;
    if (more) load_block(j + 1);
    const int kbase = j * BN;
    if (TILED) c = fmaxf(cq * p.k_descale[(size_t)bh * p.nqt + kbase / FA_FP8_TILE], kMinScale) *
                   kLog2e;
    if (!(causal && kbase > qw0 + 31)) {
      // S^T = K_j Q^T: register r of tile kt holds key kbase + 32kt +
      // 16(r/8) + 8hf + r%8 of this lane's query row.
      f32x16_t s[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        s[kt] = zero16();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint8_t* kp = &k_lds[buf][32 * kt + krow][64 * ks + 32 * hf];
          s[kt] = mfma_fp8(join(*(const u32x4_t*)kp, *(const u32x4_t*)(kp + 16)), qr[ks], s[kt]);
        }
      }
      if ((causal && kbase + BN - 1 > qw0) || kbase + BN > n_vis) {
        const int lim = (causal ? min(qrow, n_vis - 1) : n_vis - 1) - kbase - 8 * hf;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kt + 16 * (r >> 3) + (r & 7) > lim) s[kt][r] = -INFINITY;
      }
      // Block row max; the reference moves to it (and the state is rescaled)
      // only when some row's max exceeds its reference by more than
      // kHeadroom, or the reference is still -inf.
      float mx = s[0][0];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
      const float m_new = fmaxf(m_run, pair_max(mx) * c);
      if (__any(m_new > m_run + kHeadroom)) {
        const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      // e = p 448 / 2^kHeadroom = 2^(s c - m + kLog2PScale) <= 448 (p <=
      // 2^kHeadroom); the P^T operand of 64-key half kt/2 holds e rounded to
      // E4M3, byte 16(kt%2) + r of the lane's 32 = register r of tile kt.
      // The row sum accumulates e.
      const float base = ((m_run == -INFINITY) ? 0.f : m_run) - kLog2PScale;
      i32x8_t pb[NSB];
      float rs0, rs1;   // e >= 0: starting from the first pair sums is 0 + x exactly
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float e[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][4 * g + i], c, -base));
          if (kt == 0 && g == 0) {
            rs0 = e[0] + e[1];
            rs1 = e[2] + e[3];
          } else {
            rs0 += e[0] + e[1];
            rs1 += e[2] + e[3];
          }
          pb[kt >> 1][4 * (kt & 1) + g] = (int)pack_fp8x4(e[0], e[1], e[2], e[3]);
        }
      l_run += rs0 + rs1;
      // O^T += V_j^T P^T: A operand = V^T row 32dt + n, positions
      // 64sb + 32hf + 0..31 for half sb.
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint8_t* vp = &vt_lds[buf][32 * dt + n][64 * sb + 32 * hf];
          acc[dt] = mfma_fp8(join(*(const u32x4_t*)vp, *(const u32x4_t*)(vp + 16)), pb[sb],
                             acc[dt]);
        }
    }
    if (more) store_block(buf ^ 1);
    __syncthreads();
  }

  // Epilogue (l_run holds 448 / 2^kHeadroom times the row sum relative to the
  // reference): O = acc * v_descale / l_run,
  // rounded to bf16 once; LSE = (m + log2(l_run) - log2 448) ln 2.
  uint16_t* __restrict__ Oh = (uint16_t*)p.o + hoff;
  float* __restrict__ Lh = p.lse + (size_t)bh * N;
  const float lt = pair_sum(l_run);
  const float inv = lt > 0.f ? p.v_descale[bh] / lt : 0.f;
  if (qrow < N) {
    uint16_t* orow = Oh + (size_t)qrow * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2_t x = {pack_bf16(acc[dt][4 * a] * inv, acc[dt][4 * a + 1] * inv),
                     pack_bf16(acc[dt][4 * a + 2] * inv, acc[dt][4 * a + 3] * inv)};
        *(u32x2_t*)(orow + 32 * dt + 8 * a + 4 * hf) = x;
      }
    if (hf == 0)
      Lh[qrow] = lt > 0.f ? (m_run + __builtin_amdgcn_logf(lt) - kLog2PScale) * kLn2 : -INFINITY;
  }
}

template <int D, int NW, bool TILED>
void launch_fp8(unsigned grid, hipStream_t s, P8Params p) {
  static std::atomic<long long> resident{0};
  p.hg = head_group(p.causal != 0, grid,
                    resident_workgroups(fa_fwd_fp8_kernel<D, NW, TILED>, 64 * NW, resident));
  hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, NW, TILED>), dim3(grid), dim3(64 * NW), 0, s, p);
}

// Shared by fa_fwd_fp8 (one scale per head) and fa_fwd_fp8_tiled.
int fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale,
            const float* k_descale, const float* v_descale, void* o, float* lse, int B, int H,
            int N, int d, float scale, int mask_kind, const int32_t* kv_lens, void* stream,
            bool tiled) {
  if (!q || !k || !v || !q_descale || !k_descale || !v_descale || !o || !lse)
    return FA_ERR_INVALID_ARG;
  const uintptr_t al = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse;
  if (al & 15u) return FA_ERR_INVALID_ARG;
  if (((uintptr_t)q_descale | (uintptr_t)k_descale | (uintptr_t)v_descale) & 3u)
    return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
  if (mask_kind & ~(FA_MASK_CAUSAL | FA_MASK_KEY_PADDING)) return FA_ERR_INVALID_ARG;
  if ((mask_kind & FA_MASK_KEY_PADDING) && !kv_lens) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H * (((long long)N + 127) / 128) > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  if (((long long)N + 256) * d * 4 > 0xffffffffLL) return FA_ERR_INVALID_ARG;

  const bool causal = (mask_kind & FA_MASK_CAUSAL) != 0;
  const long long grid256 = (long long)B * H * ((N + 255) / 256);
  const bool big = grid256 >= (causal ? 2 : 1) * kCUs;
  const int BM = big ? 256 : 128;
  P8Params p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.q_descale = q_descale;
  p.k_descale = k_descale;
  p.v_descale = v_descale;
  p.o = o;
  p.lse = lse;
  p.kv_lens = (mask_kind & FA_MASK_KEY_PADDING) ? kv_lens : nullptr;
  p.H = H;
  p.N = N;
  p.nqb = (N + BM - 1) / BM;
  p.ascale = fabsf(scale) < kMinScale ? kMinScale : fabsf(scale);
  p.qsign = (signbit(scale) && scale != 0.f) ? 0x80808080u : 0u;
  p.causal = causal ? 1 : 0;
  p.hg = 4;
  p.nqt = (N + FA_FP8_TILE - 1) / FA_FP8_TILE;
  hipStream_t s = (hipStream_t)stream;
  const unsigned grid = (unsigned)(B * H * p.nqb);
#define FA_FP8_LAUNCH(T)                                     \
  if (d == 128) {                                            \
    if (big) launch_fp8<128, 8, T>(grid, s, p);             \
    else launch_fp8<128, 4, T>(grid, s, p);                 \
  } else {                                                   \
    if (big) launch_fp8<64, 8, T>(grid, s, p);              \
    else launch_fp8<64, 4, T>(grid, s, p);                  \
  }
  if (tiled) {
    FA_FP8_LAUNCH(true)
  } else {
    FA_FP8_LAUNCH(false)
  }
#undef FA_FP8_LAUNCH
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" int fa_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale,
                          const float* k_descale, const float* v_descale, void* o, float* lse,
                          int B, int H, int N, int d, float scale, int mask_kind,
                          const int32_t* kv_lens, void* stream) {
  return fwd_fp8(q, k, v, q_descale, k_descale, v_descale, o, lse, B, H, N, d, scale, mask_kind,
                 kv_lens, stream, false);
}

extern "C" int fa_fwd_fp8_tiled(const void* q, const void* k, const void* v,
                                const float* q_descale, const float* k_descale,
                                const float* v_descale, void* o, float* lse, int B, int H, int N,
                                int d, float scale, int mask_kind, const int32_t* kv_lens,
                                void* stream) {
  return fwd_fp8(q, k, v, q_descale, k_descale, v_descale, o, lse, B, H, N, d, scale, mask_kind,
                 kv_lens, stream, true);
}
