// Backward kernels of the exact attention library (gfx950 / MI355X), shared by
// fa_bwd.hip (head dimension 128 and the fa_bwd entry point) and
// fa_bwd_d64.hip (head dimension 64).
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
//  * fa_bwd_dkdv_kernel: keys outside, queries inside.  A workgroup owns 128
//    keys; two waves of a SIMD share 32 of them: one keeps their K rows in
//    registers, computes S = Q K^T (one key per lane) per block of 64 query
//    rows, rebuilds P from the staged LSE and accumulates dV^T += dO^T P; it
//    hands P to the other through LDS, which keeps the V rows, computes
//    dP = dO V^T, forms dS with the staged D and accumulates dK^T += Q^T dS.
//    Q and dO are staged once, row-major; the transposed operands come from
//    the transposing LDS read.  (Details above the kernel.)
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // The piece's column chunk is rotated by rg/2: a 16-byte LDS store serves
  // 8 lanes per cycle over 128 bytes of banks, and rows 4rg of 2d + 16 bytes
  // start 64 (rg odd) or 0 bytes into those 128, so without the rotation 8
  // consecutive lanes (rg = 0..7, same chunk) hit only two 16-byte positions.
  // With it they cover all eight; the transposed 8-byte stores (16 lanes,
  // 8rg bytes apart) stay conflict-free for any chunk.
  // With SPLIT, whole waves stage K, the next ones V, through one register
  // array (the choice is wave-uniform, so the buffer descriptor stays scalar).
  static_assert(!SPLIT || UNITS % 64 == 0, "staging units per wave");
  const int unit = SPLIT ? (tid < UNITS ? tid : tid - UNITS) : tid;
  const bool does_k = SPLIT ? wave < UNITS / 64 : true;
  const bool does_v = SPLIT ? (wave >= UNITS / 64 && wave < 2 * UNITS / 64) : true;
  const int rg = unit % (BN / 4), dc = (unit / (BN / 4) + rg / 2) % CPR;
  const uint32_t u_off = (uint32_t)(4 * rg) * ROWB + 16u * dc;
  u32x4_t kreg[4], vreg[4];
  auto load_block = [&](int j) {
    const int kbase = j * BN;
    const uint32_t bytes = (uint32_t)max(0, n_vis - kbase) * ROWB;
    if (SPLIT) {
      if (does_k || does_v) {
        const rsrc_t r = make_rsrc((does_k ? Kh : Vh) + (size_t)kbase * D, bytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) kreg[i] = buf_load16(r, u_off + i * ROWB);
      }
      return;
    }
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
      const u32x4_t* src = SPLIT ? kreg : vreg;
#pragma unroll
      for (int i = 0; i < 4; ++i) *(u32x4_t*)&v_lds[buf][4 * rg + i][8 * dc] = src[i];
    }
  };

  f32x16_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();
  const float c = p.c;
  const int krow = row_perm(n);
  // dP^T accumulators start from -D (every register of a lane belongs to its
  // row), so they end as dP - D.
  f32x16_t negd;
#pragma unroll
  for (int r = 0; r < 16; ++r) negd[r] = -drow;

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
      // Per 32-key tile: S^T = K_j Q^T and dP^T = V_j dO^T (key rows permuted:
      // register r of tile kt holds key kbase + 32kt + 16(r/8) + 8hf + r%8),
      // P = 2^(s c - LSE2), dS = P (dP - D) packed to bf16 as dS^T chunks
      // (chunk pc = registers 8(pc%2).. of tile pc/2 = keys 16pc + 8hf + 0..7),
      // dQ^T += K_j^T dS^T.  Order: tile 0's products; tile 1's products beside
      // tile 0's exponentials; tile 0's dQ products beside tile 1's
      // exponentials; tile 1's dQ products.
      f32x16_t s[KT], dp[KT];
      u32x4_t dsb[PC];
      const bool edge = (causal && kbase + BN - 1 > qw0) || kbase + BN > n_vis;
      const int lim = (causal ? min(qrow, n_vis - 1) : n_vis - 1) - kbase - 8 * hf;
      auto products = [&](int kt) {
        s[kt] = zero16();
        dp[kt] = negd;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4_t a = *(const u32x4_t*)&k_lds[buf][32 * kt + krow][16 * ks + 8 * hf];
          s[kt] = mfma_bf16(a, qr[ks], s[kt]);
          const u32x4_t a2 = *(const u32x4_t*)&v_lds[buf][32 * kt + krow][16 * ks + 8 * hf];
          dp[kt] = mfma_bf16(a2, dor[ks], dp[kt]);
        }
      };
      auto mask = [&](int kt) {
        if (edge) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kt + 16 * (r >> 3) + (r & 7) > lim) s[kt][r] = -INFINITY;
        }
      };
      auto dstile = [&](int kt) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int pc = 2 * kt + h, r0 = 8 * h;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r0 + 2 * w], c, -l2));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r0 + 2 * w + 1], c, -l2));
            dsb[pc][w] = pack_bf16(p0 * dp[kt][r0 + 2 * w], p1 * dp[kt][r0 + 2 * w + 1]);
          }
        }
      };
      auto dq = [&](int kt) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const int pc = 2 * kt + h;
            const u32x4_t a = *(const u32x4_t*)&kt_lds[buf][32 * dt + n][16 * pc + 8 * hf];
            acc[dt] = mfma_bf16(a, dsb[pc], acc[dt]);
          }
      };
      static_assert(KT == 2, "two key tiles per block");
      products(0);
      mask(0);
      products(1);
      dstile(0);
      mask(1);
      dq(0);
      dstile(1);
      dq(1);
    }
    if (more) store_block(buf ^ 1);
    __syncthreads();
  }

  if (qrow < N) store_rows<D>((uint16_t*)p.dq + hoff + (size_t)qrow * D, acc, p.gscale, hf);
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup = 128 keys of one (batch, head), 8 waves
// ---------------------------------------------------------------------------
// Waves g and g + 4 own keys k0 + 32g .. k0 + 32g + 31 and share a SIMD.  The
// first (role A) keeps those keys' K rows in registers, rebuilds P for each
// block of 64 query rows and accumulates dV^T += dO^T P; it hands P, rounded
// to bf16 in the layout of an MFMA operand, to the second through LDS.  The
// second (role B) keeps the V rows, computes dP = dO V^T, forms dS = P (dP - D)
// and accumulates dK^T += Q^T dS.  Role B works one query block behind role
// A, so a single barrier per block orders both the hand-over of P and the
// staging: LDS holds three stages of a query block (Q, dO, LSE, D; block i+1
// is written while role A reads block i and role B block i-1) and two P
// slots per key group.
//
// Q and dO are stored once, row-major with rows padded to 2d + 16 bytes.
// The operands of S = Q K^T and dP = dO V^T are 16-byte row reads; those of
// dV^T and dK^T (Q^T, dO^T) come from the same rows through the transposing
// LDS read (ds_read_b64_tr_b16).  Query rows are permuted within each
// 32-row tile so that both kinds of read hit 64 distinct banks: MFMA row i
// of S reads query pi(i) = 4(i%4) + 16(i/16) + 2((i/8)%2) + (i/4)%2, which
// puts query 4(r%4) + 16(r/8) + 2((r/4)%2) + h in accumulator register r of
// lane half h.  Contraction slot j (0..7) of 16-query chunk c of a tile is
// register 4c + j%4 + 8(j/4), i.e. query 4(j%4) + 16(j/4) + 2c + h: each
// transposing read covers 4 queries 4 rows apart, whose 64-byte pieces lie
// 64 bytes apart in the banks.
constexpr int kKvGroups = 4;
constexpr int kKvThreads = 128 * kKvGroups;

template <int D>
struct KvLds {
  static constexpr int BQ = 64;                         // query rows per block
  static constexpr uint32_t ROWB = D * 2;               // bytes per row in memory
  static constexpr uint32_t LROW = ROWB + 16;           // bytes per row in LDS
  static constexpr uint32_t TILE = BQ * LROW;
  static constexpr uint32_t DO = TILE;                  // offsets within a stage
  static constexpr uint32_t L = 2 * TILE;               // LSE, log2 units
  static constexpr uint32_t DV = 2 * TILE + 4 * BQ;     // -D
  static constexpr uint32_t STAGE = 2 * TILE + 8 * BQ;
  static constexpr uint32_t PSLOT = 64 * 16 * (BQ / 16);  // one wave's P chunks
  static constexpr uint32_t P = 3 * STAGE;
  static constexpr uint32_t BYTES = 3 * STAGE + 2 * kKvGroups * PSLOT;
  static constexpr int CPR = D / 8;                     // 16-byte chunks per row
  static constexpr int NCH = BQ * CPR / kKvThreads;     // chunks per thread per tensor
  static_assert(NCH * kKvThreads == BQ * CPR, "staging shape");
};

// Query (within a 32-row tile) of accumulator register r of lane half h.
__device__ __forceinline__ int kv_query(int r, int h) {
  return 4 * (r & 3) + 16 * (r >> 3) + 2 * ((r >> 2) & 1) + h;
}

template <int D>
__global__ __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv_kernel(BwdParams p) {
  using Ly = KvLds<D>;
  constexpr int BQ = Ly::BQ;
  constexpr int BK = 32 * kKvGroups;  // keys per workgroup
  constexpr int KS = D / 16;          // k-steps over d
  constexpr int DT = D / 32;          // 32-row tiles of dK^T, dV^T
  constexpr uint32_t ROWB = Ly::ROWB, LROW = Ly::LROW;

  __shared__ __attribute__((aligned(16))) uint8_t lds[Ly::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave & (kKvGroups - 1);
  const bool role_b = wave >= kKvGroups;
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
  const int kw0 = k0 + grp * 32;
  const int key = kw0 + n;
  uint16_t* dKh = (uint16_t*)p.dk + hoff;
  uint16_t* dVh = (uint16_t*)p.dv + hoff;

  if (k0 >= n_vis) {
    // No query sees these keys: their gradients are 0.
    const int rows = min(BK, N - k0);
    const u32x4_t z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < rows * Ly::CPR; i += kKvThreads) {
      const size_t off = (size_t)(k0 + i / Ly::CPR) * D + 8 * (i % Ly::CPR);
      *(u32x4_t*)(dKh + off) = z;
      *(u32x4_t*)(dVh + off) = z;
    }
    return;
  }

  // This lane's key: its K row (role A) or V row (role B) in the B-operand
  // layout of S = Q K^T / dP = dO V^T.  Keys at or past kv_len read as zero.
  u32x4_t kv[KS];
  {
    const uint32_t bytes = (uint32_t)n_vis * ROWB;
    const rsrc_t r = make_rsrc((const uint16_t*)(role_b ? p.v : p.k) + hoff, bytes);
    const uint32_t off = (uint32_t)key * ROWB + 16u * hf;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kv[ks] = buf_load16(r, off + 32u * ks);
  }

  // Staging of a query block: NCH 16-byte chunks of Q (sign-flipped when
  // scale < 0) and of dO per thread, and one LSE (threads 0..63) or -D value
  // (64..127), stored at the position its consumers read: position
  // 32t + 16h + r holds query 32t + kv_query(r, h).
  const rsrc_t rq = make_rsrc((const uint16_t*)p.q + hoff, (uint32_t)N * ROWB);
  const rsrc_t rdo = make_rsrc((const uint16_t*)p.dout + hoff, (uint32_t)N * ROWB);
  const rsrc_t rl = make_rsrc(p.lse + (size_t)bh * N, (uint32_t)N * 4u);
  const rsrc_t rd = make_rsrc(p.dps + (size_t)bh * N, (uint32_t)N * 4u);
  uint32_t g_off[Ly::NCH], l_off[Ly::NCH];
#pragma unroll
  for (int u = 0; u < Ly::NCH; ++u) {
    const int id = tid + kKvThreads * u, row = id / Ly::CPR, ch = id % Ly::CPR;
    g_off[u] = (uint32_t)row * ROWB + 16u * ch;
    l_off[u] = (uint32_t)row * LROW + 16u * ch;
  }
  const int spos = tid & (BQ - 1);
  const int sq = 32 * (spos >> 5) + kv_query(spos & 15, (spos >> 4) & 1);
  const uint32_t s_lds = (wave == 0 ? Ly::L : Ly::DV) + 4u * spos;
  u32x4_t gq[Ly::NCH], gd[Ly::NCH];
  float gs = 0.f;
  // The loads are only waited for at stage_store, at the end of the
  // iteration that issued them (the sign flip and the LSE conversion happen
  // there too).
  bool gs_ok = false;
  auto stage_load = [&](int i) {
    const uint32_t base = (uint32_t)(i * BQ) * ROWB;
#pragma unroll
    for (int u = 0; u < Ly::NCH; ++u) {
      gq[u] = buf_load16(rq, base + g_off[u]);
      gd[u] = buf_load16(rdo, base + g_off[u]);
    }
    const int row = i * BQ + sq;
    gs_ok = row < N;
    const uint32_t off = gs_ok ? 4u * (uint32_t)row : 0x80000000u;
    if (wave < 2) gs = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(wave == 0 ? rl : rd, off, 0, 0));
  };
  auto stage_store = [&](uint32_t st) {
#pragma unroll
    for (int u = 0; u < Ly::NCH; ++u) {
      *(u32x4_t*)(lds + st + l_off[u]) = gq[u] ^ p.qsign;
      *(u32x4_t*)(lds + st + Ly::DO + l_off[u]) = gd[u];
    }
    if (wave < 2) *(float*)(lds + st + s_lds) = wave == 0 ? lse_log2(gs, gs_ok) : -gs;
  };

  // Operand addresses (byte offsets within a stage's tile).  Row reads: MFMA
  // row n of tile t reads query 32t + pi(n), d elements 16ks + 8hf..+7.
  const int pin = 4 * (n & 3) + 16 * (n >> 4) + 2 * ((n >> 3) & 1) + ((n >> 2) & 1);
  const uint32_t a_row = (uint32_t)pin * LROW + 16u * hf;
  // Transposing reads: lane 16g + 4s + t reads query 4s + (g/2) (+ 32 tile
  // + 16 half + 2 chunk), d columns 16(g%2) + 4t..+3 (+ 32 dt); it receives
  // the 4 queries of d column 16(g%2) + (lane%16).
  const int tg = lane >> 4, ts = (lane >> 2) & 3, tt = lane & 3;
  const uint32_t a_tr = (uint32_t)(4 * ts + (tg >> 1)) * LROW + 32u * (tg & 1) + 8u * tt;
  const uint32_t lv_off = 4u * (16 * hf);      // LSE / D of this lane's registers
  const uint32_t p_off = Ly::P + Ly::PSLOT * (uint32_t)grp + 16u * lane;

  auto rd16 = [&](uint32_t off) { return *(const u32x4_t*)(lds + off); };
  auto rd_tr = [&](uint32_t off) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(lds + off));
    return __builtin_bit_cast(u32x2_t, v);
  };
  // A operand of dV^T / dK^T for 16-query chunk c of tile t, rows 32dt..:
  // contraction slots 0..3 from the first half of the tile, 4..7 from the
  // second.
  auto tr_operand = [&](uint32_t tile, int t, int c, int dt) {
    const uint32_t o = tile + a_tr + (uint32_t)(32 * t + 2 * c) * LROW + 64u * dt;
    const u32x2_t lo = rd_tr(o), hi = rd_tr(o + 16 * LROW);
    const u32x4_t a = {lo[0], lo[1], hi[0], hi[1]};
    return a;
  };

  f32x16_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();
  const float c = p.c;

  // Query blocks: causal -> from the block holding query k0 on; else all.
  const int qb0 = causal ? k0 / BQ : 0;
  const int nqb = (N + BQ - 1) / BQ;
  const int nblk = nqb - qb0;

  stage_load(qb0);
  stage_store(0);
  __syncthreads();

  uint32_t s_cur = 0, s_prev = 2 * Ly::STAGE, s_next = Ly::STAGE;   // stages of i, i-1, i+1
  for (int it = 0; it <= nblk; ++it) {
    const bool more = it + 1 < nblk;
    if (more) stage_load(qb0 + it + 1);
    // Block i of this role: role A block it, role B block it - 1.
    const int i = role_b ? it - 1 : it;
    const int q0 = (qb0 + i) * BQ;
    const bool active = role_b ? it > 0 : it < nblk;
    // Every key of this group is hidden, or (causal) comes after every query
    // of the block: nothing to add.
    const bool skip = kw0 >= n_vis || (causal && q0 + BQ - 1 < kw0);
    const uint32_t pslot = p_off + (uint32_t)(i & 1) * (kKvGroups * Ly::PSLOT);
    if (active && !skip && !role_b) {
      // S = Q K^T, P = 2^(s c - LSE2), dV^T += dO^T P, in the order tile 0
      // of S, tile 1 of S, P of tile 0, its dV products, P of tile 1, its dV
      // products: the exponentials of one tile run beside the MFMAs of the
      // other.  On blocks holding hidden pairs (key past kv_len, or causal
      // key after query) S starts from -inf there, so their P is 0.
      const uint32_t st = s_cur;
      f32x16_t s0 = zero16(), s1 = zero16();
      if ((causal && q0 < kw0 + 31) || kw0 + 31 >= n_vis) {
        const int thr = key >= n_vis ? (1 << 30) : (causal ? key : -1);
        const int lim = thr - q0 - hf;   // query 32t + kv_query(r, hf) hidden iff below thr
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] = kv_query(r, 0) < lim ? -INFINITY : 0.f;
          s1[r] = 32 + kv_query(r, 0) < lim ? -INFINITY : 0.f;
        }
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s0 = mfma_bf16(rd16(st + a_row + 32u * ks), kv[ks], s0);
      float lv[32];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float4 l4 = *(const float4*)(lds + st + Ly::L + lv_off + 4u * (32 * (m >> 2) + 4 * (m & 3)));
        lv[4 * m] = l4.x;
        lv[4 * m + 1] = l4.y;
        lv[4 * m + 2] = l4.z;
        lv[4 * m + 3] = l4.w;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s1 = mfma_bf16(rd16(st + a_row + 32u * LROW + 32u * ks), kv[ks], s1);
      auto p_tile = [&](const f32x16_t& sv, const float* l, int t) {
        float pr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r], c, -l[r]));
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int r0 = 4 * cc;
          const u32x4_t v = {pack_bf16(pr[r0], pr[r0 + 1]), pack_bf16(pr[r0 + 2], pr[r0 + 3]),
                             pack_bf16(pr[r0 + 8], pr[r0 + 9]),
                             pack_bf16(pr[r0 + 10], pr[r0 + 11])};
          *(u32x4_t*)(lds + pslot + 1024u * (2 * t + cc)) = v;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            acc[dt] = mfma_bf16(tr_operand(st + Ly::DO, t, cc, dt), v, acc[dt]);
        }
      };
      p_tile(s0, lv, 0);
      p_tile(s1, lv + 16, 1);
    }
    if (active && !skip && role_b) {
      // dP = dO V^T; dS = P (dP - D) with role A's P; dK^T += Q^T dS, in the
      // same tile order as role A.
      const uint32_t st = s_prev;
      // The accumulators start from -D (staged negated), so they end as dP - D.
      f32x16_t d0, d1;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float4 d4 =
            *(const float4*)(lds + st + Ly::DV + lv_off + 4u * (32 * (m >> 2) + 4 * (m & 3)));
        f32x16_t& dd = m < 4 ? d0 : d1;
        dd[4 * (m & 3)] = d4.x;
        dd[4 * (m & 3) + 1] = d4.y;
        dd[4 * (m & 3) + 2] = d4.z;
        dd[4 * (m & 3) + 3] = d4.w;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        d0 = mfma_bf16(rd16(st + Ly::DO + a_row + 32u * ks), kv[ks], d0);
      u32x4_t pb[4];
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) pb[pc] = rd16(pslot + 1024u * pc);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        d1 = mfma_bf16(rd16(st + Ly::DO + a_row + 32u * LROW + 32u * ks), kv[ks], d1);
      auto ds_tile = [&](const f32x16_t& dpv, int t) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          u32x4_t v;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int r = 4 * cc + 2 * (w & 1) + 8 * (w >> 1);
            const unsigned pp = pb[2 * t + cc][w];
            const float p0 = __uint_as_float(pp << 16), p1 = __uint_as_float(pp & 0xffff0000u);
            v[w] = pack_bf16(p0 * dpv[r], p1 * dpv[r + 1]);
          }
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            acc[dt] = mfma_bf16(tr_operand(st, t, cc, dt), v, acc[dt]);
        }
      };
      ds_tile(d0, 0);
      ds_tile(d1, 1);
    }
    if (more) stage_store(s_next);
    if (it < nblk) __syncthreads();
    const uint32_t s_free = s_prev;
    s_prev = s_cur;
    s_cur = s_next;
    s_next = s_free;
  }

  if (key < N) {
    // Q was staged with its sign flipped when scale < 0, so |scale| restores
    // scale * dS^T Q.
    if (role_b) store_rows<D>(dKh + (size_t)key * D, acc, p.ascale, hf);
    else store_rows<D>(dVh + (size_t)key * D, acc, 1.f, hf);
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
  p.nb = (p.N + 32 * kKvGroups - 1) / (32 * kKvGroups);
  const unsigned gk = (unsigned)(B * p.H * p.nb);
  static std::atomic<long long> resident_kv{0};
  p.hg = head_group(p.causal != 0, gk,
                    resident_workgroups(fa_bwd_dkdv_kernel<D>, kKvThreads, resident_kv));
  hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D>), dim3(gk), dim3(kKvThreads), 0, s, p);
  return hipGetLastError() == hipSuccess;
}

}  // namespace
