// Backward kernels of the exact attention library (gfx950 / MI355X), shared by
// fa_bwd.hip (head dimension 128 and the fa_bwd entry point) and
// fa_bwd_d64.hip (head dimension 64, compiled with MFMA results kept in
// VGPRs, which is 8-15% faster there and 2% slower at d = 128).
//
// The gradients are those of the section Backward为什么更复杂 of
// "FlashAttention算法详解：从IO瓶颈到Triton实现" (gentlecold.top), with the
// softmax scale carried by the scores:
//
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dP * P),
//     dQ = scale dS K,  dK = scale dS^T Q.
//
// As that section and §7 of the youngju.dev walkthrough describe, P is never
// read from memory: every block rebuilds it from the scores and the forward's
// per-row LSE, P = exp(scale q.k - LSE).  The row sum D is computed once per
// query row as rowsum(dO * O), which equals rowsum(dP * P) because O = P V.
//
// Two kernels, no atomics (so the result is bitwise reproducible):
//
//  * fa_bwd_dq_kernel: queries outside, keys inside, like the forward.  A
//    wave owns 32 query rows; per block of 64 keys it computes S^T = K Q^T
//    and dP^T = V dO^T (one query row per lane, keys permuted so 8
//    consecutive registers are 8 consecutive keys), rebuilds P, forms dS and
//    accumulates dQ^T += K^T dS^T with dS rounded to bf16 straight from the
//    registers.  Its prologue computes D for its rows and writes it out.
//  * fa_bwd_dkdv_kernel: keys outside, queries inside.  A wave owns 32 keys
//    (their K and V rows stay in registers as MFMA operands); per block of 64
//    query rows it computes S = Q K^T and dP = dO V^T with ONE KEY per lane,
//    rebuilds P from the staged LSE, forms dS with the staged D, and
//    accumulates dV^T += dO^T P and dK^T += Q^T dS.  Q and dO blocks are
//    staged in LDS twice: row-major (operands of S and dP) and transposed
//    (operands of dV^T and dK^T), from one set of global loads.
//
// The second kernel reads the D written by the first, so both are enqueued,
// in that order, on the caller's stream.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_api.h"
#include "fa_device.h"

namespace fa92 {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dps;            // rowsum(dP * P) per query row, [B, H, N]
  const int32_t* kv_lens;
  int H, N, nb;          // nb: work blocks per head of the launched kernel
  float c;               // |scale| * log2(e) (|scale| clamped below at 1e-30)
  float gscale;          // signed clamped scale, applied to dQ
  float ascale;          // |gscale|, applied to dK (Q is staged sign-flipped)
  unsigned qsign;        // bf16 sign flip applied to Q when scale < 0
  int causal;
  int hg;                // heads map_work visits together (head_group)
};

// Enqueues the d = 64 dQ and dK/dV kernels (defined in fa_bwd_d64.hip);
// false if a launch failed.
bool bwd_launch_d64(const BwdParams& p, int B, hipStream_t s);

}  // namespace fa92

namespace {

using namespace fa92;

__device__ __forceinline__ int visible_len(const BwdParams& p, int b) {
  if (!p.kv_lens) return p.N;
  const int kl = p.kv_lens[b];
  return kl < 0 ? 0 : (kl > p.N ? p.N : kl);
}

// LSE (natural log) -> log2 units for exp2; rows that see no key, and rows
// past N, get +inf so every rebuilt probability of theirs is exactly 0.
__device__ __forceinline__ float lse_log2(float lse, bool valid) {
  return (valid && lse > -INFINITY) ? lse * kLog2e : INFINITY;
}

// Store 32 rows x D of a transposed fp32 accumulator (lane = row, registers =
// columns 32dt + 8(r/4) + 4h + r%4) as bf16 rows, times f.
template <int D>
__device__ __forceinline__ void store_rows(uint16_t* row, const f32x16_t (&acc)[D / 32], float f,
                                           int hf) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      u32x2_t x = {pack_bf16(acc[dt][4 * a] * f, acc[dt][4 * a + 1] * f),
                   pack_bf16(acc[dt][4 * a + 2] * f, acc[dt][4 * a + 3] * f)};
      *(u32x2_t*)(row + 32 * dt + 8 * a + 4 * hf) = x;
    }
}

// ---------------------------------------------------------------------------
// dQ (and D): one workgroup = NW waves x 32 query rows of one (batch, head)
// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW >= 8 ? 2 : 1)))
void fa_bwd_dq_kernel(BwdParams p) {
  constexpr int kThreads = 64 * NW;
  constexpr int BN = 64;             // keys per block
  constexpr int BM = 32 * NW;        // query rows per workgroup
  constexpr int KS = D / 16;         // k-steps over d
  constexpr int DT = D / 32;         // 32-row tiles of dQ^T
  constexpr int KT = BN / 32;        // 32-key tiles of S^T
  constexpr int PC = BN / 16;        // 16-key chunks of dS^T
  constexpr int RLD = D + 8;         // row-major stride in LDS (elements)
  constexpr int TLD = BN + 8;        // transposed stride in LDS (elements)
  constexpr uint32_t ROWB = D * 2;   // bytes per row in device memory
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int UNITS = (BN / 4) * CPR;   // pieces of 4 rows x 8 dims per tensor
  constexpr bool SPLIT = 2 * UNITS <= kThreads;
  static_assert(SPLIT || UNITS == kThreads, "staging shape");

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][BN][RLD];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][BN][RLD];
  __shared__ __attribute__((aligned(16))) uint16_t kt_lds[2][D][TLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const bool causal = p.causal != 0;
  const int N = p.N;

  int bh, qb;
  map_work(p.nb, causal, p.hg, bh, qb);
  const int b = bh / p.H;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const uint16_t* Kh = (const uint16_t*)p.k + hoff;
  const uint16_t* Vh = (const uint16_t*)p.v + hoff;
  const int n_vis = visible_len(p, b);
  const int q0 = qb * BM;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + n;
  const int kend = causal ? min(n_vis, q0 + BM) : n_vis;
  const int nblk = (kend + BN - 1) / BN;

  // This lane's query row: Q and dO in the B-operand layout of S^T = K Q^T
  // and dP^T = V dO^T; D = dO . O; LSE in log2 units.  Rows past N read 0.
  u32x4_t qr[KS], dor[KS];
  float drow = 0.f;
  {
    const uint32_t bytes = (uint32_t)N * ROWB;
    const rsrc_t rq = make_rsrc((const uint16_t*)p.q + hoff, bytes);
    const rsrc_t rd = make_rsrc((const uint16_t*)p.dout + hoff, bytes);
    const rsrc_t ro = make_rsrc((const uint16_t*)p.o + hoff, bytes);
    const uint32_t off = (uint32_t)qrow * ROWB + 16u * hf;
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qr[ks] = buf_load16(rq, off + 32u * ks) ^ p.qsign;
      dor[ks] = buf_load16(rd, off + 32u * ks);
      const u32x4_t ov = buf_load16(ro, off + 32u * ks);
      d0 = dot_bf16x2(dor[ks][0], ov[0], dot_bf16x2(dor[ks][1], ov[1], d0));
      d1 = dot_bf16x2(dor[ks][2], ov[2], dot_bf16x2(dor[ks][3], ov[3], d1));
    }
    drow = pair_sum(d0 + d1);
  }
  const float l2 = lse_log2(qrow < N ? p.lse[(size_t)bh * N + min(qrow, N - 1)] : 0.f,
                            qrow < N);
  if (hf == 0 && qrow < N) p.dps[(size_t)bh * N + qrow] = drow;

  // Staging of key block j: pieces of 4 keys x 8 dims.  K goes to LDS
  // row-major and transposed, V row-major.  Buffer ranges end at the last
  // visible key, so hidden rows arrive as zeros (whatever memory holds).
  const int unit = SPLIT ? (tid < UNITS ? tid : tid - UNITS) : tid;
  const bool does_k = SPLIT ? tid < UNITS : true;
  const bool does_v = SPLIT ? (tid >= UNITS && tid < 2 * UNITS) : true;
  const int rg = unit % (BN / 4), dc = unit / (BN / 4);
  const uint32_t u_off = (uint32_t)(4 * rg) * ROWB + 16u * dc;
  u32x4_t kreg[4], vreg[4];
  auto load_block = [&](int j) {
    const int kbase = j * BN;
    const uint32_t bytes = (uint32_t)max(0, n_vis - kbase) * ROWB;
    if (does_k) {
      const rsrc_t rk = make_rsrc(Kh + (size_t)kbase * D, bytes);
#pragma unroll
      for (int i = 0; i < 4; ++i) kreg[i] = buf_load16(rk, u_off + i * ROWB);
    }
    if (does_v) {
      const rsrc_t rv = make_rsrc(Vh + (size_t)kbase * D, bytes);
#pragma unroll
      for (int i = 0; i < 4; ++i) vreg[i] = buf_load16(rv, u_off + i * ROWB);
    }
  };
  auto store_block = [&](int buf) {
    if (does_k) {
      u32x2_t lo[4], hi[4];
      transpose4x8(kreg, lo, hi);
#pragma unroll
      for (int i = 0; i < 4; ++i) *(u32x4_t*)&k_lds[buf][4 * rg + i][8 * dc] = kreg[i];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        *(u32x2_t*)&kt_lds[buf][8 * dc + 2 * w][4 * rg] = lo[w];
        *(u32x2_t*)&kt_lds[buf][8 * dc + 2 * w + 1][4 * rg] = hi[w];
      }
    }
    if (does_v) {
#pragma unroll
      for (int i = 0; i < 4; ++i) *(u32x4_t*)&v_lds[buf][4 * rg + i][8 * dc] = vreg[i];
    }
  };

  f32x16_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();
  const float c = p.c;
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
    const bool wave_skip = causal && (kbase > qw0 + 31);
    if (!wave_skip) {
      // S^T = K_j Q^T and dP^T = V_j dO^T, key rows permuted: register r of
      // tile kt holds key kbase + 32kt + 16(r/8) + 8hf + r%8.
      f32x16_t s[KT], dp[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        s[kt] = zero16();
        dp[kt] = zero16();
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const u32x4_t a = *(const u32x4_t*)&k_lds[buf][32 * kt + krow][16 * ks + 8 * hf];
          s[kt] = mfma_bf16(a, qr[ks], s[kt]);
          const u32x4_t a2 = *(const u32x4_t*)&v_lds[buf][32 * kt + krow][16 * ks + 8 * hf];
          dp[kt] = mfma_bf16(a2, dor[ks], dp[kt]);
        }
      if ((causal && kbase + BN - 1 > qw0) || kbase + BN > n_vis) {
        const int lim = (causal ? min(qrow, n_vis - 1) : n_vis - 1) - kbase - 8 * hf;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kt + 16 * (r >> 3) + (r & 7) > lim) s[kt][r] = -INFINITY;
      }
      // P = 2^(s c - LSE2); dS = P (dP - D), packed to bf16 as dS^T chunks
      // (chunk pc = registers 8(pc%2).. of tile pc/2 = keys 16pc + 8hf + 0..7).
      u32x4_t dsb[PC];
#pragma unroll
      for (int pc = 0; pc < PC; ++pc) {
        const int kt = pc >> 1, r0 = 8 * (pc & 1);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r0 + 2 * w], c, -l2));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r0 + 2 * w + 1], c, -l2));
          dsb[pc][w] = pack_bf16(p0 * (dp[kt][r0 + 2 * w] - drow),
                                 p1 * (dp[kt][r0 + 2 * w + 1] - drow));
        }
      }
      // dQ^T += K_j^T dS^T: A operand = K^T rows 32dt + n, keys 16pc + 8hf + 0..7.
#pragma unroll
      for (int pc = 0; pc < PC; ++pc)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const u32x4_t a = *(const u32x4_t*)&kt_lds[buf][32 * dt + n][16 * pc + 8 * hf];
          acc[dt] = mfma_bf16(a, dsb[pc], acc[dt]);
        }
    }
    if (more) store_block(buf ^ 1);
    __syncthreads();
  }

  if (qrow < N) store_rows<D>((uint16_t*)p.dq + hoff + (size_t)qrow * D, acc, p.gscale, hf);
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup = 4 waves x 32 keys of one (batch, head)
// ---------------------------------------------------------------------------
constexpr int kKvWaves = 4;

// Global -> register staging of one block of BQ query rows for the dK/dV
// kernel: pieces of 4 rows x 8 dims of Q (sign-flipped when scale < 0) and
// dO, plus LSE (log2 units) or D for one row per thread of the first 2 BQ.
struct KvStage {
  rsrc_t rq, rdo;
  rsrc_t rl, rd;      // this head's LSE and D rows (N floats each)
  uint32_t u_off;     // byte offset of this thread's piece within a block
  unsigned qsign;
  int N, tid;
  bool unit;          // this thread stages a Q/dO piece
};

// Branch-free: threads with nothing to load use an offset past the end of
// the buffer range (2^31 is beyond any accepted size), which reads zeros.
template <int D, int BQ>
__device__ __forceinline__ void kv_stage_load(const KvStage& g, int i, u32x4_t (&qreg)[4],
                                              u32x4_t (&dreg)[4], float& sreg) {
  constexpr uint32_t ROWB = D * 2;
  constexpr uint32_t kOut = 0x80000000u;
  const uint32_t off = g.unit ? (uint32_t)(i * BQ) * ROWB + g.u_off : kOut;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    qreg[t] = buf_load16(g.rq, off + t * ROWB) ^ g.qsign;
    dreg[t] = buf_load16(g.rdo, off + t * ROWB);
  }
  const int row = i * BQ + (g.tid % BQ);
  const bool ok = row < g.N;
  const float l = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
      g.rl, (ok && g.tid < BQ) ? 4u * row : kOut, 0, 0));
  const float d = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
      g.rd, (ok && g.tid >= BQ && g.tid < 2 * BQ) ? 4u * row : kOut, 0, 0));
  sreg = g.tid < BQ ? lse_log2(l, ok) : d;
}

// One block of BQ query rows for one wave's 32 keys: S = Q K^T and
// dP = dO V^T (one key per lane, query rows permuted so register r of tile qt
// holds query q0 + 32qt + 16(r/8) + 8hf + r%8), P = 2^(s c - LSE2),
// dS = P (dP - D), then dV^T += dO^T P and dK^T += Q^T dS.  EDGE: the block
// holds hidden pairs (key past kv_len, or causal key after query); the other
// blocks skip the mask.  The next block's global loads are issued after the
// softmax, when the scores no longer occupy registers.  The body is one
// straight-line region (the staging loads are branch-free).
template <int D, int BQ, bool EDGE>
__device__ __forceinline__ void kv_block(
    const uint16_t (*q_rows)[D + 8], const uint16_t (*do_rows)[D + 8],
    const uint16_t (*q_cols)[BQ + 8], const uint16_t (*do_cols)[BQ + 8], const float* l_vec,
    const float* d_vec, const u32x4_t (&kr)[D / 16], const u32x4_t (&vr)[D / 16],
    f32x16_t (&dva)[D / 32], f32x16_t (&dka)[D / 32], const KvStage& g, int inext,
    u32x4_t (&qreg)[4], u32x4_t (&dreg)[4], float& sreg, int q0, int key, int n_vis,
    bool causal, float c, int n, int hf, int qperm) {
  constexpr int KS = D / 16, DT = D / 32, QT = BQ / 32, PC = BQ / 16;
  f32x16_t s[QT], dp[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    s[qt] = zero16();
    dp[qt] = zero16();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4_t a = *(const u32x4_t*)&q_rows[32 * qt + qperm][16 * ks + 8 * hf];
      s[qt] = mfma_bf16(a, kr[ks], s[qt]);
      const u32x4_t a2 = *(const u32x4_t*)&do_rows[32 * qt + qperm][16 * ks + 8 * hf];
      dp[qt] = mfma_bf16(a2, vr[ks], dp[qt]);
    }
  }
  if constexpr (EDGE) {
    const bool hidden_key = key >= n_vis;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = q0 + 32 * qt + 16 * (r >> 3) + 8 * hf + (r & 7);
        if (hidden_key || (causal && key > qi)) s[qt][r] = -INFINITY;
      }
  }
  // Chunk pc of 16 queries = registers 8(pc%2).. of tile pc/2.
  u32x4_t pb[PC], dsb[PC];
#pragma unroll
  for (int pc = 0; pc < PC; ++pc) {
    const int qt = pc >> 1, r0 = 8 * (pc & 1);
    const float4* lp = (const float4*)&l_vec[16 * pc + 8 * hf];
    const float4* dpp = (const float4*)&d_vec[16 * pc + 8 * hf];
    const float4 la = lp[0], lb = lp[1], da = dpp[0], db = dpp[1];
    const float lv[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
    const float dv[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qt][r0 + 2 * w], c, -lv[2 * w]));
      const float p1 =
          __builtin_amdgcn_exp2f(__builtin_fmaf(s[qt][r0 + 2 * w + 1], c, -lv[2 * w + 1]));
      pb[pc][w] = pack_bf16(p0, p1);
      dsb[pc][w] = pack_bf16(p0 * (dp[qt][r0 + 2 * w] - dv[2 * w]),
                             p1 * (dp[qt][r0 + 2 * w + 1] - dv[2 * w + 1]));
    }
  }
  // Past the last block the loads read zeros and rows past N; unused.
  kv_stage_load<D, BQ>(g, inext, qreg, dreg, sreg);
  // A operands: rows 32dt + n of the transposed tiles, queries 16pc + 8hf + 0..7.
#pragma unroll
  for (int pc = 0; pc < PC; ++pc)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const u32x4_t a = *(const u32x4_t*)&do_cols[32 * dt + n][16 * pc + 8 * hf];
      dva[dt] = mfma_bf16(a, pb[pc], dva[dt]);
      const u32x4_t a2 = *(const u32x4_t*)&q_cols[32 * dt + n][16 * pc + 8 * hf];
      dka[dt] = mfma_bf16(a2, dsb[pc], dka[dt]);
    }
}

template <int D>
__global__ __launch_bounds__(64 * kKvWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_bwd_dkdv_kernel(BwdParams p) {
  constexpr int kThreads = 64 * kKvWaves;
  constexpr int BK = 32 * kKvWaves;  // keys per workgroup
  constexpr int BQ = 64;             // query rows per block
  constexpr int KS = D / 16;         // k-steps over d
  constexpr int DT = D / 32;         // 32-row tiles of dK^T, dV^T
  constexpr int RLD = D + 8;
  constexpr int TLD = BQ + 8;
  constexpr uint32_t ROWB = D * 2;
  constexpr int CPR = D / 8;
  constexpr int UNITS = (BQ / 4) * CPR;
  static_assert(UNITS <= kThreads && 2 * BQ <= kThreads, "staging shape");

  __shared__ __attribute__((aligned(16))) uint16_t q_lds[2][BQ][RLD];
  __shared__ __attribute__((aligned(16))) uint16_t do_lds[2][BQ][RLD];
  __shared__ __attribute__((aligned(16))) uint16_t qt_lds[2][D][TLD];
  __shared__ __attribute__((aligned(16))) uint16_t dot_lds[2][D][TLD];
  __shared__ __attribute__((aligned(16))) float l_lds[2][BQ];   // LSE, log2 units
  __shared__ __attribute__((aligned(16))) float d_lds[2][BQ];   // D

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const bool causal = p.causal != 0;
  const int N = p.N;

  int bh, kb;
  map_work(p.nb, false, p.hg, bh, kb);   // causal: key block 0 (the most query blocks) first
  const int b = bh / p.H;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const int n_vis = visible_len(p, b);
  const int k0 = kb * BK;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + n;
  uint16_t* dKh = (uint16_t*)p.dk + hoff;
  uint16_t* dVh = (uint16_t*)p.dv + hoff;

  if (k0 >= n_vis) {
    // No query sees these keys: their gradients are 0.
    const int rows = min(BK, N - k0);
    const u32x4_t z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < rows * CPR; i += kThreads) {
      const size_t off = (size_t)(k0 + i / CPR) * D + 8 * (i % CPR);
      *(u32x4_t*)(dKh + off) = z;
      *(u32x4_t*)(dVh + off) = z;
    }
    return;
  }

  // This lane's key: K and V rows in the B-operand layout of S = Q K^T and
  // dP = dO V^T.  Keys at or past kv_len read as zero.
  u32x4_t kr[KS], vr[KS];
  {
    const uint32_t bytes = (uint32_t)n_vis * ROWB;
    const rsrc_t rk = make_rsrc((const uint16_t*)p.k + hoff, bytes);
    const rsrc_t rv = make_rsrc((const uint16_t*)p.v + hoff, bytes);
    const uint32_t off = (uint32_t)key * ROWB + 16u * hf;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kr[ks] = buf_load16(rk, off + 32u * ks);
      vr[ks] = buf_load16(rv, off + 32u * ks);
    }
  }

  // Query blocks: causal -> from the block holding query k0 on; else all.
  const int qb0 = causal ? k0 / BQ : 0;
  const int nqb = (N + BQ - 1) / BQ;

  // Staging of query block i: pieces of 4 rows x 8 dims of Q and dO, stored
  // row-major and transposed; LSE (log2 units) and D for its rows.
  const bool st_unit = tid < UNITS;
  const int rg = tid % (BQ / 4), dc = tid / (BQ / 4);
  const uint32_t u_off = (uint32_t)(4 * rg) * ROWB + 16u * dc;
  const rsrc_t rq = make_rsrc((const uint16_t*)p.q + hoff, (uint32_t)N * ROWB);
  const rsrc_t rdo = make_rsrc((const uint16_t*)p.dout + hoff, (uint32_t)N * ROWB);
  const float* Lh = p.lse + (size_t)bh * N;
  const float* Dh = p.dps + (size_t)bh * N;
  u32x4_t qreg[4], dreg[4];
  float sreg = 0.f;
  KvStage g;
  g.rq = rq;
  g.rdo = rdo;
  g.rl = make_rsrc(Lh, (uint32_t)N * 4u);
  g.rd = make_rsrc(Dh, (uint32_t)N * 4u);
  g.u_off = u_off;
  g.qsign = p.qsign;
  g.N = N;
  g.tid = tid;
  g.unit = st_unit;
  auto store_block = [&](int buf) {
    if (st_unit) {
      u32x2_t lo[4], hi[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) *(u32x4_t*)&q_lds[buf][4 * rg + t][8 * dc] = qreg[t];
      transpose4x8(qreg, lo, hi);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        *(u32x2_t*)&qt_lds[buf][8 * dc + 2 * w][4 * rg] = lo[w];
        *(u32x2_t*)&qt_lds[buf][8 * dc + 2 * w + 1][4 * rg] = hi[w];
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) *(u32x4_t*)&do_lds[buf][4 * rg + t][8 * dc] = dreg[t];
      transpose4x8(dreg, lo, hi);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        *(u32x2_t*)&dot_lds[buf][8 * dc + 2 * w][4 * rg] = lo[w];
        *(u32x2_t*)&dot_lds[buf][8 * dc + 2 * w + 1][4 * rg] = hi[w];
      }
    }
    if (tid < BQ) l_lds[buf][tid] = sreg;
    else if (tid < 2 * BQ) d_lds[buf][tid - BQ] = sreg;
  };

  f32x16_t dka[DT], dva[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dka[dt] = zero16();
    dva[dt] = zero16();
  }
  const float c = p.c;
  const int qperm = row_perm(n);

  if (qb0 < nqb) {
    kv_stage_load<D, BQ>(g, qb0, qreg, dreg, sreg);
    store_block(0);
  }
  __syncthreads();

  for (int i = qb0; i < nqb; ++i) {
    const int buf = (i - qb0) & 1;
    const int q0 = i * BQ;
    // Every key of this wave is hidden, or (causal) comes after every query
    // of the block: nothing to add, only the staging goes on.
    const bool wave_skip = kw0 >= n_vis || (causal && q0 + BQ - 1 < kw0);
    const bool edge = (causal && q0 < kw0 + 31) || (kw0 + 31 >= n_vis);
    if (wave_skip)
      kv_stage_load<D, BQ>(g, i + 1, qreg, dreg, sreg);
    else if (edge)
      kv_block<D, BQ, true>(q_lds[buf], do_lds[buf], qt_lds[buf], dot_lds[buf], l_lds[buf],
                            d_lds[buf], kr, vr, dva, dka, g, i + 1, qreg, dreg, sreg, q0, key,
                            n_vis, causal, c, n, hf, qperm);
    else
      kv_block<D, BQ, false>(q_lds[buf], do_lds[buf], qt_lds[buf], dot_lds[buf], l_lds[buf],
                             d_lds[buf], kr, vr, dva, dka, g, i + 1, qreg, dreg, sreg, q0, key,
                             n_vis, causal, c, n, hf, qperm);
    if (i + 1 < nqb) store_block(buf ^ 1);
    __syncthreads();
  }

  if (key < N) {
    store_rows<D>(dVh + (size_t)key * D, dva, 1.f, hf);
    // Q was staged with its sign flipped when scale < 0, so |scale| restores
    // scale * dS^T Q.
    store_rows<D>(dKh + (size_t)key * D, dka, p.ascale, hf);
  }
}

// dQ and D: 256-row workgroups (8 waves) when they fill the chip at least
// twice over for causal masks (once otherwise), else 128 rows (4 waves);
// then dK and dV: 128 keys per workgroup.  Both on stream s, in that order;
// false if a launch failed (the dK/dV kernel is then not enqueued).
template <int D, int NW>
void launch_dq(unsigned grid, hipStream_t s, BwdParams p) {
  static std::atomic<long long> resident{0};
  p.hg = head_group(p.causal != 0, grid,
                    resident_workgroups(fa_bwd_dq_kernel<D, NW>, 64 * NW, resident));
  hipLaunchKernelGGL((fa_bwd_dq_kernel<D, NW>), dim3(grid), dim3(64 * NW), 0, s, p);
}

template <int D>
bool launch_bwd(BwdParams p, int B, hipStream_t s) {
  const long long grid256 = (long long)B * p.H * ((p.N + 255) / 256);
  const bool big = grid256 >= (p.causal ? 2 : 1) * kCUs;
  const int BM = big ? 256 : 128;
  p.nb = (p.N + BM - 1) / BM;
  const unsigned gq = (unsigned)(B * p.H * p.nb);
  if (big) launch_dq<D, 8>(gq, s, p);
  else launch_dq<D, 4>(gq, s, p);
  if (hipGetLastError() != hipSuccess) return false;
  p.nb = (p.N + 32 * kKvWaves - 1) / (32 * kKvWaves);
  const unsigned gk = (unsigned)(B * p.H * p.nb);
  static std::atomic<long long> resident_kv{0};
  p.hg = head_group(p.causal != 0, gk,
                    resident_workgroups(fa_bwd_dkdv_kernel<D>, 64 * kKvWaves, resident_kv));
  hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D>), dim3(gk), dim3(64 * kKvWaves), 0, s, p);
  return hipGetLastError() == hipSuccess;
}

}  // namespace
