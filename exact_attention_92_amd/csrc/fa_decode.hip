// Attention decode over a paged KV cache for gfx950 (MI355X): the split and
// combine kernels and the fa_decode_paged entry point of include/fa_api.h.
//
// One query token per request attends to its n cached tokens, which live in
// a pool of fixed-size blocks reached through the request's block table
// (§7 of "FlashAttention 完整解析" on freezetheflame.cc).  The work is one
// pass over the cached keys and values, 4*d bytes per token and head against
// 4*d FLOPs: bandwidth-bound, so no matrix cores -- coalesced 16-byte loads
// and VALU dot products.
//
//  * Split kernel: one workgroup (4 waves) per (request, head, chunk of 512
//    tokens).  A lane owns 8 head dimensions of one token per step, so a
//    wave reads 64 x 16 contiguous bytes (d/8 lanes per token row) of K and
//    of V per step, with non-temporal loads; steps are unrolled four deep so
//    enough loads are in flight.  The block table is read once per step (a wave's tokens share a
//    block).  Each lane keeps the online-softmax state (running max m,
//    running sum l, unnormalised accumulator) of the tokens it saw, in log2
//    units ("FlashAttention算法详解" section Online Softmax); the states of the
//    lanes, then of the waves, are merged with the rescaling identity of §6.3
//    of the youngju.dev walkthrough, and the chunk's (m, l, acc) is written to
//    the workspace.
//  * Combine kernel: per (request, head), merges the chunks' states the same
//    way, writes O (bf16) and LSE.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "fa_api.h"
#include "fa_device.h"

// Scratch of fa_decode_paged_noalloc: the per-chunk partial results between
// its two kernels live here instead of in a caller workspace.  Every GPU the
// library runs on holds its own copy until the process ends; the host side
// reaches it only through the device address hipGetSymbolAddress returns.
static __device__ __align__(256) float scratch[FA_DECODE_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

using namespace fa92;

constexpr int kChunk = 512;        // tokens per split
// Cache policy of the K/V loads: non-temporal ("nt").  Every cached row is
// read exactly once per call, so its lines should not displace anything;
// measured +12% over the default policy.
constexpr int kStreamLoad = 2;
constexpr int kDecThreads = 256;   // 4 waves

struct DecParams {
  const void* q;
  const void* kp;
  const void* vp;
  const int32_t* tables;
  const int32_t* lens;
  void* o;
  float* lse;
  float* ws;
  int H, bs, max_blocks, num_blocks, nsplit;
  float c;   // scale * log2(e)
};

__device__ __forceinline__ int seq_len(const DecParams& p, int b) {
  const int n = p.lens[b];
  const int cap = p.max_blocks * p.bs;
  return n < 0 ? 0 : (n > cap ? cap : n);
}

// Merge online-softmax state (m2, l2, a2) into (m, l, a).
template <int NA>
__device__ __forceinline__ void merge(float& m, float& l, float (&a)[NA], float m2, float l2,
                                      const float (&a2)[NA]) {
  const float mn = fmaxf(m, m2);
  const float f1 = (mn == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
  const float f2 = (mn == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
  l = l * f1 + l2 * f2;
#pragma unroll
  for (int i = 0; i < NA; ++i) a[i] = a[i] * f1 + a2[i] * f2;
  m = mn;
}

__device__ __forceinline__ float shfl_xor(float x, int mask) {
  return __shfl_xor(x, mask, 64);
}

template <int D>
__global__ __launch_bounds__(kDecThreads) void fa_decode_split_kernel(DecParams p) {
  constexpr int LPT = D / 8;            // lanes per token row (16-byte pieces)
  constexpr int TPS = 64 / LPT;         // tokens per wave step
  constexpr int UNROLL = 4;
  constexpr uint32_t ROWB = D * 2;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n = seq_len(p, b);
  const int t0 = split * kChunk;
  if (t0 >= n) return;                  // the combine kernel never reads this chunk
  const int t1 = min(n, t0 + kChunk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int piece = lane % LPT, slot_in_step = lane / LPT;

  // This lane's 8 query values (fp32), dims 8*piece .. 8*piece+7.
  float qv[8];
  {
    const u32x4_t w = *(const u32x4_t*)((const uint16_t*)p.q + ((size_t)b * p.H + h) * D + 8 * piece);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qv[2 * i] = __uint_as_float(w[i] << 16);
      qv[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  const int32_t* table = p.tables + (size_t)b * p.max_blocks;
  const size_t head_block = (size_t)p.bs * D;          // elements of one (block, head)
  const uint32_t block_bytes = (uint32_t)(p.bs * ROWB);

  float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;

  const int nsteps = (t1 - t0 + TPS - 1) / TPS;
  // Wave w takes steps w, w + 4, w + 8, ...; UNROLL steps per round.
  for (int s0 = wave; s0 < nsteps; s0 += 4 * UNROLL) {
    u32x4_t kr[UNROLL], vr[UNROLL];
    int tok[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int st = s0 + 4 * u;
      const int tfirst = t0 + st * TPS;                  // wave-uniform
      tok[u] = tfirst + slot_in_step;
      kr[u] = u32x4_t{0u, 0u, 0u, 0u};
      vr[u] = u32x4_t{0u, 0u, 0u, 0u};
      if (st < nsteps) {
        const int j = tfirst / p.bs;
        const int phys = table[j];
        const bool ok = phys >= 0 && phys < p.num_blocks;
        const size_t base = ((size_t)(ok ? phys : 0) * p.H + h) * head_block;
        const rsrc_t rk = make_rsrc((const uint16_t*)p.kp + base, ok ? block_bytes : 0u);
        const rsrc_t rv = make_rsrc((const uint16_t*)p.vp + base, ok ? block_bytes : 0u);
        const uint32_t off = (uint32_t)(tok[u] - j * p.bs) * ROWB + 16u * piece;
        kr[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, kStreamLoad);
        vr[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, kStreamLoad);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      float sdot = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sdot = __builtin_fmaf(qv[2 * i], __uint_as_float(kr[u][i] << 16), sdot);
        sdot = __builtin_fmaf(qv[2 * i + 1], __uint_as_float(kr[u][i] & 0xffff0000u), sdot);
      }
#pragma unroll
      for (int off = 1; off < LPT; off <<= 1) sdot += shfl_xor(sdot, off);
      // Slots past the sequence end (the rest of its last block) may hold
      // anything, NaN included: their score is -inf and their V row 0.
      const bool valid = tok[u] < t1;
      if (!valid) vr[u] = u32x4_t{0u, 0u, 0u, 0u};
      const float s2 = valid ? sdot * p.c : -INFINITY;
      const float mn = fmaxf(m, s2);
      const float alpha = (mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m - mn);
      const float pr = (mn == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s2 - mn);
      l = l * alpha + pr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = acc[2 * i] * alpha + pr * __uint_as_float(vr[u][i] << 16);
        acc[2 * i + 1] = acc[2 * i + 1] * alpha + pr * __uint_as_float(vr[u][i] & 0xffff0000u);
      }
      m = mn;
    }
  }

  // Merge the token slots of the wave (lanes piece + LPT * k).
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
    float a2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a2[i] = shfl_xor(acc[i], off);
    merge<8>(m, l, acc, shfl_xor(m, off), shfl_xor(l, off), a2);
  }
  // Merge the 4 waves through LDS: wave w writes (m, l, acc[D]); wave 0 merges.
  __shared__ float sm[4], sl[4];
  __shared__ __attribute__((aligned(16))) float sa[4][D];
  if (lane < LPT) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sa[wave][8 * lane + i] = acc[i];
    if (lane == 0) {
      sm[wave] = m;
      sl[wave] = l;
    }
  }
  __syncthreads();
  if (wave == 0 && lane < LPT) {
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      float a2[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) a2[i] = sa[w][8 * lane + i];
      merge<8>(m, l, acc, sm[w], sl[w], a2);
    }
    float* out = p.ws + (((size_t)b * p.H + h) * p.nsplit + split) * (D + 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[8 * lane + i] = acc[i];
    if (lane == 0) {
      out[D] = m;
      out[D + 1] = l;
    }
  }
}

// One workgroup of D threads per (request, head): thread t owns dim t.
template <int D>
__global__ __launch_bounds__(D) void fa_decode_combine_kernel(DecParams p) {
  const int bh = blockIdx.x;
  const int b = bh / p.H;
  const int t = threadIdx.x;
  const int n = seq_len(p, b);
  const int ns = (n + kChunk - 1) / kChunk;
  const float* ws = p.ws + (size_t)bh * p.nsplit * (D + 2);
  float m = -INFINITY;
  for (int s = 0; s < ns; ++s) m = fmaxf(m, ws[s * (D + 2) + D]);
  float l = 0.f, a = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float ms = ws[s * (D + 2) + D];
    const float f = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - m);
    l += ws[s * (D + 2) + D + 1] * f;
    a += ws[s * (D + 2) + t] * f;
  }
  const float o = l > 0.f ? a / l : 0.f;
  ((uint16_t*)p.o)[(size_t)bh * D + t] = (uint16_t)(pack_bf16(o, 0.f) & 0xffffu);
  if (t == 0) p.lse[bh] = l > 0.f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
}

int nsplit_of(int bs, int max_blocks) {
  const long long cap = (long long)bs * max_blocks;
  return (int)((cap + kChunk - 1) / kChunk);
}

}  // namespace

extern "C" size_t fa_decode_paged_workspace_bytes(int B, int H, int d, int block_size,
                                                  int max_blocks_per_seq) {
  if (B < 1 || H < 1 || (d != 64 && d != 128) || block_size < 8 || max_blocks_per_seq < 1)
    return 0;
  return (size_t)B * H * nsplit_of(block_size, max_blocks_per_seq) * (d + 2) * sizeof(float);
}

namespace {

// Argument checks shared by both decode entry points (everything but the
// workspace).
int check_decode(const void* q, const void* k_pool, const void* v_pool,
                 const int32_t* block_tables, const int32_t* seq_lens, const void* o,
                 const float* lse, int B, int H, int d, int block_size, int max_blocks_per_seq,
                 int num_blocks, float scale) {
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !o || !lse)
    return FA_ERR_INVALID_ARG;
  if (((uintptr_t)q | (uintptr_t)k_pool | (uintptr_t)v_pool | (uintptr_t)o) & 15u)
    return FA_ERR_INVALID_ARG;
  if (((uintptr_t)block_tables | (uintptr_t)seq_lens | (uintptr_t)lse) & 3u)
    return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || max_blocks_per_seq < 1 || num_blocks < 1) return FA_ERR_INVALID_ARG;
  if (block_size < 8 || block_size % 8 != 0 || block_size > 65536) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const long long nsplit = nsplit_of(block_size, max_blocks_per_seq);
  if (B > 65535 || H > 65535 || nsplit > 0x7fffffffLL ||
      (long long)block_size * max_blocks_per_seq > 0x7fffffffLL)
    return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// Enqueues the split and combine kernels with `workspace` as their scratch
// (arguments already checked).
int launch_decode(const void* q, const void* k_pool, const void* v_pool,
                  const int32_t* block_tables, const int32_t* seq_lens, void* o, float* lse,
                  float* workspace, int B, int H, int d, int block_size, int max_blocks_per_seq,
                  int num_blocks, float scale, void* stream) {
  DecParams p;
  p.q = q;
  p.kp = k_pool;
  p.vp = v_pool;
  p.tables = block_tables;
  p.lens = seq_lens;
  p.o = o;
  p.lse = lse;
  p.ws = workspace;
  p.H = H;
  p.bs = block_size;
  p.max_blocks = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.nsplit = nsplit_of(block_size, max_blocks_per_seq);
  p.c = scale * kLog2e;
  hipStream_t s = (hipStream_t)stream;
  const dim3 g1((unsigned)p.nsplit, (unsigned)H, (unsigned)B);
  if (d == 128) hipLaunchKernelGGL((fa_decode_split_kernel<128>), g1, dim3(kDecThreads), 0, s, p);
  else hipLaunchKernelGGL((fa_decode_split_kernel<64>), g1, dim3(kDecThreads), 0, s, p);
  if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  const dim3 g2((unsigned)(B * H));
  if (d == 128) hipLaunchKernelGGL((fa_decode_combine_kernel<128>), g2, dim3(128), 0, s, p);
  else hipLaunchKernelGGL((fa_decode_combine_kernel<64>), g2, dim3(64), 0, s, p);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Device address of the current GPU's copy of `scratch`, looked up once per
// device (with that device current) and kept; nullptr if the runtime cannot
// give it.
constexpr int kMaxDevices = 256;
std::atomic<float*> scratch_ptr[kMaxDevices];
std::mutex scratch_mu;

float* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  float* ptr = scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  ptr = scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!ptr) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) {
      (void)hipGetLastError();
      return nullptr;
    }
    ptr = (float*)addr;
    scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

}  // namespace

extern "C" int fa_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_tables, const int32_t* seq_lens, void* o,
                               float* lse, float* workspace, int B, int H, int d, int block_size,
                               int max_blocks_per_seq, int num_blocks, float scale,
                               void* stream) {
  if (!workspace || ((uintptr_t)workspace & 3u)) return FA_ERR_INVALID_ARG;
  const int st = check_decode(q, k_pool, v_pool, block_tables, seq_lens, o, lse, B, H, d,
                              block_size, max_blocks_per_seq, num_blocks, scale);
  if (st != FA_OK) return st;
  return launch_decode(q, k_pool, v_pool, block_tables, seq_lens, o, lse, workspace, B, H, d,
                       block_size, max_blocks_per_seq, num_blocks, scale, stream);
}

extern "C" int fa_decode_paged_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                       const int32_t* block_tables, const int32_t* seq_lens,
                                       void* o, float* lse, int B, int H, int d, int block_size,
                                       int max_blocks_per_seq, int num_blocks, float scale,
                                       void* stream) {
  const int st = check_decode(q, k_pool, v_pool, block_tables, seq_lens, o, lse, B, H, d,
                              block_size, max_blocks_per_seq, num_blocks, scale);
  if (st != FA_OK) return st;
  if (fa_decode_paged_workspace_bytes(B, H, d, block_size, max_blocks_per_seq) >
      FA_DECODE_NOALLOC_SCRATCH_BYTES)
    return FA_ERR_SCRATCH;
  float* ws = scratch_on_current_device();
  if (!ws) return FA_ERR_HIP;
  return launch_decode(q, k_pool, v_pool, block_tables, seq_lens, o, lse, ws, B, H, d,
                       block_size, max_blocks_per_seq, num_blocks, scale, stream);
}
