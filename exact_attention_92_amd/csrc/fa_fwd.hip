// Exact attention forward for gfx950 (MI355X): bf16 and fp32 kernels plus the
// C ABI declared in include/fa_api.h.
//
// The method is the IO-aware online-softmax forward of "FlashAttention算法详解：
// 从IO瓶颈到Triton实现" (gentlecold.top), sections Online Softmax and
// FlashAttention Forward流程: a block of query rows keeps a running row max m,
// a running row sum l and an unnormalised output accumulator acc; for every
// block of keys it computes the scores, moves m up, rescales l and acc by
// alpha = exp(m_old - m_new), adds the block's exp(score - m_new) to l and
// exp(score - m_new) V to acc, and divides by l once at the end (the
// FlashAttention-2 order of §4.3 of "FlashAttention 完整解析" on
// freezetheflame.cc: queries outside, keys inside, normalise last).
//
// Mapping to CDNA4 (design notes in the repository describe the choices):
//
//  * One workgroup = 4 wavefronts = one block of 32*QW*4 query rows of one
//    (batch, head).  Each wave owns 32*QW query rows; the wave's rows are the
//    N dimension of a 32x32 MFMA tile.  K/V blocks of 64 keys are shared by
//    the 4 waves through LDS (double buffered, prefetched into registers one
//    block ahead).
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: the accumulator then holds ONE query per lane
//    (lane % 32) and 16 keys per lane, so the softmax row statistics are
//    per-lane scalars plus one exchange between lanes l and l^32.
//  * The K rows fed to the MFMA are permuted (bits 2 and 3 of the row index
//    swapped) so that each lane's 8 consecutive accumulator registers hold 8
//    CONSECUTIVE keys.  Those registers, rounded to bf16, are directly the B
//    operand of O^T = V^T P^T; V is stored transposed in LDS so the A operand
//    is one 16-byte LDS read per lane.  P never leaves registers.
//  * Scores are kept in log2 units (scale * log2(e) folded into one FMA) and
//    exponentiated with v_exp_f32 (a native 2^x).  The probabilities are
//    rounded to bf16 for the P V product.  Two row sums are kept: one over
//    the rounded values (v_dot2c_f32_bf16 against 1.0) normalises O, so the
//    weights applied to V sum to exactly 1; the fp32 one gives LSE.
//  * The running max is only moved when a block's max exceeds it by more than
//    TAU (log2 units); the exponentials are then bounded by 2^TAU and most
//    blocks skip the accumulator rescale.  Any reference point gives the
//    same softmax (the rescaling identity of the online-softmax section of
//    the youngju.dev walkthrough, §6.3), so this is exact up to rounding.
//  * Causal: key blocks above the workgroup's last row are never loaded;
//    a wave skips the blocks above its own rows; only blocks that cross the
//    diagonal, the key-padding edge or the sequence end are masked
//    element-wise ("Causal Mask怎么处理" on the gentlecold.top page).
//  * Workgroups are dispatched round-robin over the 8 XCDs; the block index
//    is remapped so that consecutive work items of one head land on one XCD
//    (shared L2 for that head's K/V), and causal query blocks run heaviest
//    first.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_api.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;              // keys per block (bf16 kernel)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;         // max-move threshold, log2 units
constexpr float kMinScale = 1e-30f;

__device__ __forceinline__ f32x16_t mfma_bf16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma_f32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Value of lane (l ^ 32) combined with lane l's own value.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2_t));
}

// acc + (lo + hi) of a packed bf16 pair, in fp32 (v_dot2c_f32_bf16 with 1.0).
__device__ __forceinline__ float sum_bf16x2(unsigned pair, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair),
                                         __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
}

// Row of K that MFMA row m reads: bits 2 and 3 of m swapped.  With it, the
// accumulator register r of lane-half h holds key 16*(r/8) + 8*h + (r%8) of
// each 32-key tile.
__device__ __forceinline__ int k_row_perm(int m) {
  return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Maps the linear workgroup id to (head, query block).  Workgroups are
// dispatched round-robin over 8 XCDs; when the grid divides evenly, XCD x
// gets the contiguous logical range [x*G/8, (x+1)*G/8).  Within a head,
// causal query blocks are visited from the last (heaviest) to the first.
__device__ __forceinline__ void map_block(int nqb, bool causal, int& bh, int& qb) {
  const int G = gridDim.x;
  const int w = blockIdx.x;
  const int L = (G % 8 == 0) ? (w % 8) * (G / 8) + w / 8 : w;
  bh = L / nqb;
  const int r = L - bh * nqb;
  qb = causal ? (nqb - 1 - r) : r;
}

struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* kv_lens;
  int H, N, nqb;
  float c;          // |scale| * log2(e), >= kMinScale * log2(e)
  unsigned qsign;   // sign flip applied to Q when scale < 0
  int causal;
};

// ---------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------
#ifndef FA_WAVES_PER_EU
#define FA_WAVES_PER_EU 2
#endif

template <int D, int QW>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(FA_WAVES_PER_EU)))
void fa_fwd_bf16_kernel(Params p) {
  constexpr int BM = 32 * QW * kWaves;
  constexpr int KS = D / 16;        // MFMA k-steps over d for S^T
  constexpr int DT = D / 32;        // 32-row tiles of O^T
  constexpr int KT = kBN / 32;      // 32-key tiles of S^T
  constexpr int PC = kBN / 16;      // 16-key chunks of P^T
  constexpr int KLD = D + 8;        // K row stride in LDS (elements)
  constexpr int VLD = kBN + 8;      // V^T row stride in LDS (elements)
  constexpr int KU = kBN * (D / 8) / kThreads;   // 16-byte K pieces per thread
  constexpr int VUNITS = (kBN / 4) * (D / 8);    // 4-key x 8-d V pieces
  static_assert(KU >= 1 && VUNITS <= kThreads, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kBN][KLD];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][D][VLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const bool causal = p.causal != 0;
  const int N = p.N;

  int bh, qb;
  map_block(p.nqb, causal, bh, qb);
  const int b = bh / p.H;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ Qh = (const uint16_t*)p.q + hoff;
  const uint16_t* __restrict__ Kh = (const uint16_t*)p.k + hoff;
  const uint16_t* __restrict__ Vh = (const uint16_t*)p.v + hoff;

  int n_vis = N;
  if (p.kv_lens) {
    const int kl = p.kv_lens[b];
    n_vis = kl < 0 ? 0 : (kl > N ? N : kl);
  }
  const int q0 = qb * BM;
  const int qw0 = q0 + wave * 32 * QW;
  int kend = n_vis;
  if (causal) kend = min(kend, q0 + BM);
  const int nblk = (kend + kBN - 1) / kBN;

  // Q rows of this wave, in the B-operand layout of S^T = K Q^T.
  u32x4_t qr[QW][KS];
#pragma unroll
  for (int qt = 0; qt < QW; ++qt) {
    const int row = qw0 + 32 * qt + n;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (row < N) x = *(const u32x4_t*)(Qh + (size_t)row * D + 16 * ks + 8 * hf);
      qr[qt][ks] = x ^ p.qsign;
    }
  }

  float m_run[QW], l_run[QW], le_run[QW];
  f32x16_t acc[QW][DT];
#pragma unroll
  for (int qt = 0; qt < QW; ++qt) {
    m_run[qt] = -INFINITY;
    l_run[qt] = 0.f;
    le_run[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qt][dt][r] = 0.f;
  }

  u32x4_t kreg[KU];
  u32x4_t vreg[4];

  // Global -> registers for key block j.  K pieces are row-major 16-byte
  // chunks (coalesced).  V pieces are 4 keys x 8 dims so they can be written
  // transposed with 8-byte LDS stores.  Keys >= N read nothing (zero); V rows
  // of hidden padding keys are zeroed so that 0 * garbage cannot occur.
  auto load_block = [&](int j) {
    const int kbase = j * kBN;
    const bool full = kbase + kBN <= n_vis;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int unit = tid + u * kThreads;
      const int key = unit / (D / 8);
      const int ch = unit % (D / 8);
      const int gk = kbase + key;
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (full || gk < N) x = *(const u32x4_t*)(Kh + (size_t)gk * D + 8 * ch);
      kreg[u] = x;
    }
    if (tid < VUNITS) {
      const int kg = tid % (kBN / 4);
      const int dc = tid / (kBN / 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int gk = kbase + 4 * kg + i;
        u32x4_t x = {0u, 0u, 0u, 0u};
        if (full || gk < n_vis) x = *(const u32x4_t*)(Vh + (size_t)gk * D + 8 * dc);
        vreg[i] = x;
      }
    }
  };

  auto store_block = [&](int buf) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int unit = tid + u * kThreads;
      const int key = unit / (D / 8);
      const int ch = unit % (D / 8);
      *(u32x4_t*)&k_lds[buf][key][8 * ch] = kreg[u];
    }
    if (tid < VUNITS) {
      const int kg = tid % (kBN / 4);
      const int dc = tid / (kBN / 4);
#pragma unroll
      for (int pw = 0; pw < 4; ++pw) {
        const unsigned a0 = vreg[0][pw], a1 = vreg[1][pw], a2 = vreg[2][pw], a3 = vreg[3][pw];
        u32x2_t lo = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
        u32x2_t hi = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
        *(u32x2_t*)&vt_lds[buf][8 * dc + 2 * pw][4 * kg] = lo;
        *(u32x2_t*)&vt_lds[buf][8 * dc + 2 * pw + 1][4 * kg] = hi;
      }
    }
  };

  if (nblk > 0) {
    load_block(0);
    store_block(0);
  }
  __syncthreads();

  const int krow = k_row_perm(n);
  const float c = p.c;

  for (int j = 0; j < nblk; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < nblk;
    if (more) load_block(j + 1);
    const int kbase = j * kBN;
    const bool wave_skip = causal && (kbase > qw0 + 32 * QW - 1);
    if (!wave_skip) {
      // S^T = K_j Q^T
      f32x16_t s[QW][KT];
#pragma unroll
      for (int qt = 0; qt < QW; ++qt)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[qt][kt][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const u32x4_t a = *(const u32x4_t*)&k_lds[buf][32 * kt + krow][16 * ks + 8 * hf];
#pragma unroll
          for (int qt = 0; qt < QW; ++qt) s[qt][kt] = mfma_bf16(a, qr[qt][ks], s[qt][kt]);
        }
      }

      const bool need_mask = (causal && kbase + kBN - 1 > qw0) || (kbase + kBN > n_vis);
      if (need_mask) {
#pragma unroll
        for (int qt = 0; qt < QW; ++qt) {
          const int qrow = qw0 + 32 * qt + n;
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kbase + 32 * kt + 16 * (r >> 3) + 8 * hf + (r & 7);
              const bool hide = (causal && key > qrow) || key >= n_vis;
              if (hide) s[qt][kt][r] = -INFINITY;
            }
        }
      }

      u32x4_t pb[QW][PC];
#pragma unroll
      for (int qt = 0; qt < QW; ++qt) {
        float mx = s[qt][0][0];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qt][kt][r]);
        mx = pair_max(mx);
        const float mt = mx * c;                  // block max, log2 units
        const bool upd = mt > m_run[qt] + kTau;   // false while nothing is visible
        float alpha = 1.f;
        if (__any(upd)) {
          const float m_new = upd ? mt : m_run[qt];
          alpha = upd ? __builtin_amdgcn_exp2f(m_run[qt] - m_new) : 1.f;
          m_run[qt] = m_new;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[qt][dt][r] *= alpha;
        }
        const float base = (m_run[qt] == -INFINITY) ? 0.f : m_run[qt];
        float re0 = 0.f, re1 = 0.f;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qt][kt][r], c, -base));
            const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qt][kt][r + 1], c, -base));
            s[qt][kt][r] = e0;
            s[qt][kt][r + 1] = e1;
            re0 += e0;
            re1 += e1;
          }
        // Two row sums: the fp32 one gives LSE; the one over the
        // bf16-rounded probabilities (the weights that actually multiply V)
        // normalises O, so those weights sum to exactly 1.
        float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
        for (int pc = 0; pc < PC; ++pc) {
          const int kt = pc >> 1, r0 = 8 * (pc & 1);
          u32x4_t x;
#pragma unroll
          for (int w = 0; w < 4; ++w)
            x[w] = pack_bf16(s[qt][kt][r0 + 2 * w], s[qt][kt][r0 + 2 * w + 1]);
          pb[qt][pc] = x;
          rs0 = sum_bf16x2(x[0], sum_bf16x2(x[1], rs0));
          rs1 = sum_bf16x2(x[2], sum_bf16x2(x[3], rs1));
        }
        l_run[qt] = l_run[qt] * alpha + (rs0 + rs1);
        le_run[qt] = le_run[qt] * alpha + (re0 + re1);
      }

      // O^T += V_j^T P^T
#pragma unroll
      for (int pc = 0; pc < PC; ++pc) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const u32x4_t a = *(const u32x4_t*)&vt_lds[buf][32 * dt + n][16 * pc + 8 * hf];
#pragma unroll
          for (int qt = 0; qt < QW; ++qt) acc[qt][dt] = mfma_bf16(a, pb[qt][pc], acc[qt][dt]);
        }
      }
    }
    if (more) store_block((j + 1) & 1);
    __syncthreads();
  }

  // Epilogue: O = acc / l (rounded to bf16 once), LSE = (m + log2 l) * ln 2.
  uint16_t* __restrict__ Oh = (uint16_t*)p.o + hoff;
  float* __restrict__ Lh = p.lse + (size_t)bh * N;
#pragma unroll
  for (int qt = 0; qt < QW; ++qt) {
    const float lt = pair_sum(l_run[qt]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int qrow = qw0 + 32 * qt + n;
    if (qrow < N) {
      uint16_t* orow = Oh + (size_t)qrow * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          u32x2_t x = {pack_bf16(acc[qt][dt][4 * a] * inv, acc[qt][dt][4 * a + 1] * inv),
                       pack_bf16(acc[qt][dt][4 * a + 2] * inv, acc[qt][dt][4 * a + 3] * inv)};
          *(u32x2_t*)(orow + 32 * dt + 8 * a + 4 * hf) = x;
        }
      const float le = pair_sum(le_run[qt]);
      if (hf == 0)
        Lh[qrow] = lt > 0.f ? (m_run[qt] + __builtin_amdgcn_logf(le)) * kLn2 : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel (v_mfma_f32_32x32x2_f32; no narrowing anywhere)
// ---------------------------------------------------------------------------
constexpr int kBN32 = 32;

template <int D>
__global__ __launch_bounds__(kThreads) void fa_fwd_f32_kernel(Params p) {
  constexpr int BM = 32 * kWaves;
  constexpr int KS = D / 2;         // k-steps of the 32x32x2 MFMA
  constexpr int DT = D / 32;
  constexpr int KLD = D + 4;
  constexpr int KU = kBN32 * (D / 4) / kThreads;  // 16-byte pieces per thread (K and V each)
  static_assert(KU >= 1, "tile shape");

  __shared__ __attribute__((aligned(16))) float k_lds[kBN32][KLD];
  __shared__ __attribute__((aligned(16))) float v_lds[kBN32][KLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const bool causal = p.causal != 0;
  const int N = p.N;

  int bh, qb;
  map_block(p.nqb, causal, bh, qb);
  const int b = bh / p.H;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const float* __restrict__ Qh = (const float*)p.q + hoff;
  const float* __restrict__ Kh = (const float*)p.k + hoff;
  const float* __restrict__ Vh = (const float*)p.v + hoff;

  int n_vis = N;
  if (p.kv_lens) {
    const int kl = p.kv_lens[b];
    n_vis = kl < 0 ? 0 : (kl > N ? N : kl);
  }
  const int q0 = qb * BM;
  const int qw0 = q0 + wave * 32;
  int kend = n_vis;
  if (causal) kend = min(kend, q0 + BM);
  const int nblk = (kend + kBN32 - 1) / kBN32;
  const float qs = p.qsign ? -1.f : 1.f;

  const int qrow = qw0 + n;
  float qr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qr[ks] = qrow < N ? qs * Qh[(size_t)qrow * D + 2 * ks + hf] : 0.f;

  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  const float c = p.c;

  for (int j = 0; j < nblk; ++j) {
    const int kbase = j * kBN32;
    __syncthreads();  // previous block fully consumed
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int unit = tid + u * kThreads;
      const int key = unit / (D / 4);
      const int ch = unit % (D / 4);
      const int gk = kbase + key;
      u32x4_t kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
      if (gk < N) kx = *(const u32x4_t*)(Kh + (size_t)gk * D + 4 * ch);
      if (gk < n_vis) vx = *(const u32x4_t*)(Vh + (size_t)gk * D + 4 * ch);
      *(u32x4_t*)&k_lds[key][4 * ch] = kx;
      *(u32x4_t*)&v_lds[key][4 * ch] = vx;
    }
    __syncthreads();
    if (causal && kbase > qw0 + 31) continue;

    f32x16_t s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = mfma_f32(k_lds[n][2 * ks + hf], qr[ks], s);

    if ((causal && kbase + kBN32 - 1 > qw0) || (kbase + kBN32 > n_vis)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kbase + 8 * (r >> 2) + 4 * hf + (r & 3);
        if ((causal && key > qrow) || key >= n_vis) s[r] = -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = pair_max(mx);
    const float mt = mx * c;
    const bool upd = mt > m_run + kTau;
    float alpha = 1.f;
    if (__any(upd)) {
      const float m_new = upd ? mt : m_run;
      alpha = upd ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
    }
    const float base = (m_run == -INFINITY) ? 0.f : m_run;
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -base));
      rs += s[r];
    }
    l_run = l_run * alpha + rs;
    // O^T += V^T P^T: the 2-key chunk r pairs key 8(r/4)+(r%4) (lanes 0-31)
    // with key 8(r/4)+(r%4)+4 (lanes 32-63), exactly the keys of register r.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + (r & 3) + 4 * hf;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma_f32(v_lds[key][32 * dt + n], s[r], acc[dt]);
    }
  }

  float* __restrict__ Oh = (float*)p.o + hoff;
  float* __restrict__ Lh = p.lse + (size_t)bh * N;
  const float lt = pair_sum(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qrow < N) {
    float* orow = Oh + (size_t)qrow * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float4 x = make_float4(acc[dt][4 * a] * inv, acc[dt][4 * a + 1] * inv,
                               acc[dt][4 * a + 2] * inv, acc[dt][4 * a + 3] * inv);
        *(float4*)(orow + 32 * dt + 8 * a + 4 * hf) = x;
      }
    if (hf == 0) Lh[qrow] = lt > 0.f ? (m_run + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
#ifndef FA_QW
#define FA_QW 1
#endif
constexpr int kQW = FA_QW;  // 32-query tiles per wave in the bf16 kernel

int check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
               int B, int H, int N, int d, float scale, int mask_kind, const int32_t* kv_lens,
               int bm) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  const uintptr_t al = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse;
  if (al & 15u) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
  if (mask_kind & ~(FA_MASK_CAUSAL | FA_MASK_KEY_PADDING)) return FA_ERR_INVALID_ARG;
  if ((mask_kind & FA_MASK_KEY_PADDING) && !kv_lens) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const long long nqb = ((long long)N + bm - 1) / bm;
  if ((long long)B * H * nqb > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

Params make_params(const void* q, const void* k, const void* v, void* o, float* lse, int H, int N,
                   int nqb, float scale, int mask_kind, const int32_t* kv_lens) {
  Params p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.kv_lens = (mask_kind & FA_MASK_KEY_PADDING) ? kv_lens : nullptr;
  p.H = H;
  p.N = N;
  p.nqb = nqb;
  float a = fabsf(scale);
  if (a < kMinScale) a = kMinScale;
  p.c = a * kLog2e;
  p.qsign = signbit(scale) && scale != 0.f ? 0x80008000u : 0u;
  p.causal = (mask_kind & FA_MASK_CAUSAL) ? 1 : 0;
  return p;
}

}  // namespace

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int N, int d, float scale, int mask_kind, const int32_t* kv_lens,
                      void* stream) {
  constexpr int BM = 32 * kQW * kWaves;
  const int st = check_args(q, k, v, o, lse, B, H, N, d, scale, mask_kind, kv_lens, BM);
  if (st != FA_OK) return st;
  const int nqb = (N + BM - 1) / BM;
  const Params p = make_params(q, k, v, o, lse, H, N, nqb, scale, mask_kind, kv_lens);
  const dim3 grid((unsigned)(B * H * nqb)), block(kThreads);
  hipStream_t s = (hipStream_t)stream;
  if (d == 128)
    hipLaunchKernelGGL((fa_fwd_bf16_kernel<128, kQW>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((fa_fwd_bf16_kernel<64, kQW>), grid, block, 0, s, p);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                          int H, int N, int d, float scale, int mask_kind, const int32_t* kv_lens,
                          void* stream) {
  constexpr int BM = 32 * kWaves;
  const int st = check_args(q, k, v, o, lse, B, H, N, d, scale, mask_kind, kv_lens, BM);
  if (st != FA_OK) return st;
  const int nqb = (N + BM - 1) / BM;
  const Params p = make_params(q, k, v, o, lse, H, N, nqb, scale, mask_kind, kv_lens);
  const dim3 grid((unsigned)(B * H * nqb)), block(kThreads);
  hipStream_t s = (hipStream_t)stream;
  if (d == 128)
    hipLaunchKernelGGL((fa_fwd_f32_kernel<128>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((fa_fwd_f32_kernel<64>), grid, block, 0, s, p);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension (d must be 64 or 128)";
    case FA_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}
