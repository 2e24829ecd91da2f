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
// Mapping to CDNA4 (the design notes of the repository give the measurements
// behind each choice):
//
//  * One workgroup = 8 wavefronts = one block of 256 query rows of one
//    (batch, head); each wave owns 32 rows, the N dimension of a 32x32 MFMA
//    tile.  Two waves share each SIMD, so one wave's MFMAs overlap the
//    other's softmax.  Blocks of 64 keys (128 for d <= 64) are staged
//    through LDS, double buffered: raw buffer loads bring block j+1 into
//    registers while block j is computed (rows past the end read as zero).
//    LDS operand reads are issued well ahead of their MFMAs (scheduling
//    hints), since an LDS round trip under load spans about ten MFMA issue
//    intervals.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: the accumulator holds ONE query row per lane
//    (lane % 32) and 16 keys per lane, so the softmax row statistics are
//    per-lane scalars plus one exchange between lanes l and l^32
//    (v_permlane32_swap).
//  * The K rows fed to the MFMA are permuted (bits 2 and 3 of the row index
//    swapped) so each lane's 8 consecutive accumulator registers hold 8
//    CONSECUTIVE keys.  Rounded to bf16 they are directly the B operand of
//    O^T = V^T P^T; P never leaves registers.  V is transposed on its way
//    into LDS (v_perm_b32 regrouping, 8-byte stores) so the A operand of
//    every P V MFMA is one 16-byte ds_read_b128; on gfx950 that read moves
//    twice the bytes per clock of the ds_read_b64_tr_b16 transpose read.
//  * Scores are kept in log2 units (scale * log2(e) folded into one FMA) and
//    exponentiated with v_exp_f32 (a native 2^x).  The probabilities are
//    rounded to bf16 for the P V product.  Two row sums are kept: one over
//    the rounded values (v_dot2c_f32_bf16 against 1.0) normalises O, so the
//    weights applied to V sum to exactly 1; the fp32 one gives LSE.
//  * The running max is a reference point that moves only when it must: a
//    wave's first block sets it from the block's row max; later blocks
//    exponentiate against it directly, and only when a row sum shows a
//    probability above 2^20 (or an infinite one) is the block redone with a
//    fresh row max and the state rescaled.  Any reference point gives the
//    same softmax (the rescaling identity of the online-softmax section of
//    the youngju.dev walkthrough, §6.3), so this is exact up to rounding; it
//    removes the per-block row-max reduction and almost every rescale.
//  * Causal: key blocks above the workgroup's last row are never loaded;
//    a wave skips the blocks above its own rows; only blocks that cross the
//    diagonal, the key-padding edge or the sequence end are masked
//    element-wise ("Causal Mask怎么处理" on the gentlecold.top page).
//  * Workgroups are dispatched round-robin over the 8 XCDs; the work items
//    (head, query block) are ordered so that all items of one head land on
//    one XCD (shared L2 for that head's K/V) and causal query blocks run
//    heaviest first.  For contiguous self-attention the grid is capped at
//    the workgroups the chip holds at once and each workgroup loops over its
//    items in a snake order.
//  * One kernel template serves three entry points: contiguous
//    self-attention (fa_fwd), the general layout with N_q != N_k, a sliding
//    window and arbitrary strides (fa_fwd_general), and packed sequences of
//    different lengths (fa_fwd_varlen); head dimensions 32 to 256.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>

#include "fa_api.h"
#include "fa_device.h"

namespace {

using namespace fa92;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kOverflowSum = 1048576.f;  // 2^20: largest block row sum kept on the fast path
constexpr float kTau = 8.0f;         // fp32 kernel: max-move threshold, log2 units

__device__ __forceinline__ f32x16_t mfma_f32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row of K that MFMA row m reads (row_perm): with it, the accumulator
// register r of lane-half h holds key 16*(r/8) + 8*h + (r%8) of each 32-key
// tile, so 8 consecutive registers are 8 consecutive keys.
__device__ __forceinline__ int k_row_perm(int m) { return row_perm(m); }

// Scheduling hint for a run of NM MFMAs, each fed by one LDS operand read:
// issue AHEAD reads first, then alternate MFMA and read.  LDS round trips
// under load are ~10 MFMA issue intervals, so the reads must run well ahead.
#ifndef FA_READ_AHEAD
#define FA_READ_AHEAD 6
#endif
template <int NM, int AHEAD>
__device__ __forceinline__ void mfma_read_ahead() {
  if (AHEAD > 0) __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i + AHEAD < NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// Heads an XCD visits together for launches whose items are not all
// resident (head_group in fa_device.h chooses 8 for causal launches that fit
// the chip at once: measured +19-23% at B = 4, H = 16, N = 1024, d = 64/128;
// on grids larger than the chip 8 heads gave the same speed with 1.4x the
// HBM traffic).
struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* kv_lens;
  int H, N, nqb;    // N: query rows (and keys, unless the general layout is used)
  int items;        // work items (head, query block) = B * H * nqb
  int hg;           // heads an XCD visits together (map_work), 4 or 8
  float c;          // |scale| * log2(e), >= kMinScale * log2(e)
  unsigned qsign;   // sign flip applied to Q when scale < 0
  int causal;
  // General layout only: key count, key position of query row 0 (Nk - Nq),
  // sliding window (-1: none), batch/head strides (elements) and row
  // strides (bytes for q, k, v; elements for o).
  int Nk, off, window;
  long long qbs, qhs, kbs, khs, vbs, vhs, obs, ohs;
  unsigned qrs, krs, vrs, ors;
  // Packed variable-length sequences only: sequence b owns query rows
  // [cu_q[b], cu_q[b+1]) of total_q and key rows [cu_k[b], cu_k[b+1]) of
  // total_k; lse is [H, total_q].
  const int32_t* cu_q;
  const int32_t* cu_k;
  long long total_q, total_k;
};

// ---------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------
#ifndef FA_WAVES_PER_EU
#define FA_WAVES_PER_EU 2
#endif
#ifndef FA_V_PREFETCH
#define FA_V_PREFETCH 8
#endif


// MODE 0: contiguous self-attention [B, H, N, d]; every length, offset and
// stride is a compile-time constant or N.  MODE 1 (general): N_q != N_k with
// the queries at the last N_q key positions, sliding window, arbitrary
// batch/head/row strides.  MODE 2 (varlen): MODE 1 over packed sequences
// whose boundaries are read from cu_q / cu_k.
// d = 256 needs about 300 live registers: one wave per SIMD.
template <int D, int NW, int MODE>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(D > 128 ? 1 : FA_WAVES_PER_EU)))
void fa_fwd_bf16_kernel(Params p) {
  constexpr bool GEN = MODE != 0;
  constexpr bool VL = MODE == 2;
  constexpr int kThreads = 64 * NW;
  // Keys per block: 128 for d <= 64, where the softmax work per MFMA is
  // largest and halving the per-block loop, barrier and staging overhead
  // pays; 64 otherwise (the register budget).
  constexpr int BN = D <= 64 ? 128 : 64;
  constexpr int BM = 32 * NW;       // query rows per workgroup
  constexpr int KS = D / 16;        // MFMA k-steps over d for S^T
  constexpr int DT = D / 32;        // 32-row tiles of O^T
  constexpr int KT = BN / 32;       // 32-key tiles of S^T
  constexpr int PC = BN / 16;       // 16-key chunks of P^T
  constexpr int KLD = D + 8;        // K row stride in LDS (elements)
  constexpr int VLD = BN + 8;       // V^T row stride in LDS (elements)
  constexpr uint32_t ROWB = D * 2;  // bytes per row in device memory
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int KUNITS = BN * CPR;           // 16-byte K pieces per block
  constexpr int KU = (KUNITS + kThreads - 1) / kThreads;   // per thread
  constexpr bool KFULL = KUNITS % kThreads == 0;           // every thread has KU pieces
  constexpr int VUNITS = (BN / 4) * CPR;     // V pieces of 4 keys x 8 dims
  constexpr int VU = (VUNITS + kThreads - 1) / kThreads;   // per thread
  static_assert(D % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][BN][KLD];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][D][VLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const bool causal = p.causal != 0;
  // Work items: this workgroup takes items in rounds, snaking (odd rounds
  // visit the positions in reverse) so heavy and light causal blocks even out;
  // with 8 | G and 8 | P the items of a round keep their XCD lane.
  const int P = gridDim.x, G = p.items;
  const bool lanes8 = !VL && G % 8 == 0 && P % 8 == 0;
  const int L8 = lanes8 ? 8 : 1;
  const int lx = blockIdx.x % L8, mx = blockIdx.x / L8, Pm = P / L8, Gm = G / L8;
  for (int round = 0;; ++round) {
    const int idx = round * Pm + ((round & 1) ? Pm - 1 - mx : mx);
    if (idx >= Gm) break;
    const int w_item = idx * L8 + lx;
    if (round > 0) __syncthreads();
    int N = p.N;

    int bh, qb;
    map_work(p.nqb, causal, p.hg, VL, w_item, p.items, bh, qb);
    const int b = bh / p.H;
    int Nk = GEN ? p.Nk : N;
    int off = GEN ? p.off : 0;                // key position of query row 0
    long long qr0 = 0, kr0 = 0;               // varlen: first packed row of the sequence
    if (VL) {
      // Boundaries clamped into the packed tensors, so any cu values stay in bounds.
      const long long q_s = min(max((long long)p.cu_q[b], 0LL), p.total_q);
      const long long q_e = min(max((long long)p.cu_q[b + 1], q_s), p.total_q);
      const long long k_s = min(max((long long)p.cu_k[b], 0LL), p.total_k);
      const long long k_e = min(max((long long)p.cu_k[b + 1], k_s), p.total_k);
      N = (int)(q_e - q_s);
      Nk = (int)(k_e - k_s);
      off = Nk - N;
      qr0 = q_s;
      kr0 = k_s;
      if (qb * (32 * NW) >= N) continue;      // whole workgroup past the sequence's rows
    }
    const int W = GEN ? p.window : -1;        // keys visible before a query's own position
    const uint32_t QRB = GEN ? p.qrs : ROWB;  // row strides in bytes
    const uint32_t KRB = GEN ? p.krs : ROWB;
    const uint32_t VRB = GEN ? p.vrs : ROWB;
    const size_t hoff = (size_t)bh * (size_t)N * D;
    const int hh = bh - b * p.H;
    const uint16_t* Qh = (const uint16_t*)p.q +
                         (GEN ? b * p.qbs + hh * p.qhs + qr0 * (QRB / 2) : (long long)hoff);
    const uint16_t* Kh = (const uint16_t*)p.k +
                         (GEN ? b * p.kbs + hh * p.khs + kr0 * (KRB / 2) : (long long)hoff);
    const uint16_t* Vh = (const uint16_t*)p.v +
                         (GEN ? b * p.vbs + hh * p.vhs + kr0 * (VRB / 2) : (long long)hoff);

    int n_vis = Nk;
    if (p.kv_lens) {
      const int kl = p.kv_lens[b];
      n_vis = kl < 0 ? 0 : (kl > Nk ? Nk : kl);
    }
    const int q0 = qb * BM;
    const int qw0 = q0 + wave * 32;
    const int kend = causal ? min(n_vis, q0 + BM + off) : n_vis;
    const int nblk = (kend + BN - 1) / BN;
    // With a window, blocks entirely before the first row's window are skipped.
    const int jstart = (W >= 0) ? max(0, q0 + off - W) / BN : 0;

    // Q rows of this wave in the B-operand layout of S^T = K Q^T.  Rows past N
    // lie outside the buffer range and read as zero.
    u32x4_t qr[KS];
    {
      const rsrc_t rq = make_rsrc(Qh, (uint32_t)N * QRB);
      const uint32_t qoff = (uint32_t)(qw0 + n) * QRB + 16u * hf;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qr[ks] = buf_load16(rq, qoff + 32u * ks) ^ p.qsign;
    }

    // Global -> register staging of key block j.  K: row-major 16-byte
    // pieces.  V: pieces of 4 keys x 8 dims, written to LDS transposed.  The
    // buffer range of V ends at the last visible key, so hidden V rows arrive
    // as zeros; K rows past N read zero.
    uint32_t k_off[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int unit = tid + u * kThreads;
      // A thread without a piece reads past every buffer range (zeros).
      k_off[u] = (KFULL || unit < KUNITS) ? (uint32_t)(unit / CPR) * KRB + 16u * (unit % CPR)
                                          : 0x80000000u;
    }
    bool v_unit[VU];
    int vkg[VU], vdc[VU];
    uint32_t v_off[VU];
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int unit = tid + u * kThreads;
      v_unit[u] = unit < VUNITS;
      vkg[u] = unit % (BN / 4);
      vdc[u] = unit / (BN / 4);
      v_off[u] = (uint32_t)(4 * vkg[u]) * VRB + 16u * vdc[u];
    }
    u32x4_t kreg[KU], vreg[VU][4];
    auto load_block = [&](int j) {
      const int kbase = j * BN;
      const rsrc_t rk =
          make_rsrc(Kh + (size_t)kbase * (KRB / 2), (uint32_t)max(0, Nk - kbase) * KRB);
      const rsrc_t rv =
          make_rsrc(Vh + (size_t)kbase * (VRB / 2), (uint32_t)max(0, n_vis - kbase) * VRB);
#pragma unroll
      for (int u = 0; u < KU; ++u) kreg[u] = buf_load16(rk, k_off[u]);
#pragma unroll
      for (int u = 0; u < VU; ++u) {
        if (v_unit[u]) {
#pragma unroll
          for (int i = 0; i < 4; ++i) vreg[u][i] = buf_load16(rv, v_off[u] + i * VRB);
        }
      }
    };
    auto store_block = [&](int buf) {
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int unit = tid + u * kThreads;
        if (KFULL || unit < KUNITS) *(u32x4_t*)&k_lds[buf][unit / CPR][8 * (unit % CPR)] = kreg[u];
      }
#pragma unroll
      for (int u = 0; u < VU; ++u) {
        if (v_unit[u]) {
          // Dword w of key i holds dims 8*vdc + 2w, +1: regroup into
          // (keys 0-3 of dim 2w) and (keys 0-3 of dim 2w+1).
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const unsigned a0 = vreg[u][0][w], a1 = vreg[u][1][w], a2 = vreg[u][2][w],
                           a3 = vreg[u][3][w];
            const u32x2_t lo = {__builtin_amdgcn_perm(a1, a0, 0x05040100u),
                                __builtin_amdgcn_perm(a3, a2, 0x05040100u)};
            const u32x2_t hi = {__builtin_amdgcn_perm(a1, a0, 0x07060302u),
                                __builtin_amdgcn_perm(a3, a2, 0x07060302u)};
            *(u32x2_t*)&vt_lds[buf][8 * vdc[u] + 2 * w][4 * vkg[u]] = lo;
            *(u32x2_t*)&vt_lds[buf][8 * vdc[u] + 2 * w + 1][4 * vkg[u]] = hi;
          }
        }
      }
    };

    float m_run = -INFINITY;   // reference max, log2 units (one query row per lane)
    float l_run = 0.f;         // row sum of the bf16-rounded probabilities (normalises O)
    float le_run = 0.f;        // row sum of the fp32 probabilities (gives LSE)
    f32x16_t acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
    const float c = p.c;
    const int krow = k_row_perm(n);
    bool have_ref = false;   // wave-uniform: m_run was set by a full pass

    // p = 2^(s*c - base), packed to bf16 as P^T (chunk pc = registers
    // 8(pc%2)..+7 of key tile pc/2 = keys 16pc + 8hf + 0..7) with both row
    // sums; the scores are left intact.
    auto exps = [&](const f32x16_t (&s)[KT], u32x4_t (&pb)[PC], float base, float& re,
                    float& rs) {
      float re0, re1, rs0 = 0.f, rs1 = 0.f;   // p >= 0: the fp32 sums start at the first p
#pragma unroll
      for (int pc = 0; pc < PC; ++pc) {
        const int kt = pc >> 1, r0 = 8 * (pc & 1);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r0 + 2 * w], c, -base));
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r0 + 2 * w + 1], c, -base));
          re0 = (pc == 0 && w == 0) ? e0 : re0 + e0;
          re1 = (pc == 0 && w == 0) ? e1 : re1 + e1;
          pb[pc][w] = pack_bf16(e0, e1);
        }
        rs0 = sum_bf16x2(pb[pc][0], sum_bf16x2(pb[pc][1], rs0));
        rs1 = sum_bf16x2(pb[pc][2], sum_bf16x2(pb[pc][3], rs1));
      }
      re = re0 + re1;
      rs = rs0 + rs1;
    };

    if (jstart < nblk) {
      load_block(jstart);
      store_block(0);
    }
    __syncthreads();

    for (int j = jstart; j < nblk; ++j) {
      const int buf = (j - jstart) & 1;
      const bool more = j + 1 < nblk;
      if (more) load_block(j + 1);
      const int kbase = j * BN;
      const bool wave_skip = (causal && (kbase > qw0 + 31 + off)) ||
                             (W >= 0 && kbase + BN - 1 < qw0 + off - W);
      if (!wave_skip) {
        // S^T = K_j Q^T with K rows permuted (row 32kt + krow feeds MFMA row n).
        f32x16_t s[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            const u32x4_t a = *(const u32x4_t*)&k_lds[buf][32 * kt + krow][16 * ks + 8 * hf];
            s[kt] = mfma_bf16(a, qr[ks], s[kt]);
          }
        mfma_read_ahead<KS * KT, FA_READ_AHEAD>();
        // The first V^T operands are requested now, so they arrive while the
        // softmax runs.
        constexpr int VPRE = FA_V_PREFETCH < PC * DT ? FA_V_PREFETCH : PC * DT;
        u32x4_t vpre[VPRE > 0 ? VPRE : 1];
#pragma unroll
        for (int i = 0; i < VPRE; ++i)
          vpre[i] = *(const u32x4_t*)&vt_lds[buf][32 * (i % DT) + n][16 * (i / DT) + 8 * hf];
        // Register r of key tile kt holds key kbase + 32kt + 16(r/8) + 8hf + r%8.
        if ((causal && kbase + BN - 1 > qw0 + off) || kbase + BN > n_vis ||
            (W >= 0 && kbase < qw0 + 31 + off - W)) {
          const int qrow = qw0 + n;
          const int lim = (causal ? min(qrow + off, n_vis - 1) : n_vis - 1) - kbase - 8 * hf;
          const int lim_lo = (W >= 0) ? qrow + off - W - kbase - 8 * hf : -BN;
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int idx = 32 * kt + 16 * (r >> 3) + (r & 7);
              if (idx > lim || idx < lim_lo) s[kt][r] = -INFINITY;
            }
        }

        // Exponentials against the reference max.  A wave's first block, or a
        // block whose fp32 row sum shows a probability above 2^20 (or an
        // infinite one), takes the full path: block row max, move the
        // reference, rescale the state, redo the exponentials.
        u32x4_t pb[PC];
        float re = 0.f, rs = 0.f;
        bool full = !have_ref;
        if (!full) {
          exps(s, pb, m_run, re, rs);
          full = __any(!(re <= kOverflowSum));
        }
        if (full) {
          float mx = s[0][0];
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
          const float m_new = fmaxf(m_run, pair_max(mx) * c);
          const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
          l_run *= alpha;
          le_run *= alpha;
          m_run = m_new;
          have_ref = true;
          exps(s, pb, (m_new == -INFINITY) ? 0.f : m_new, re, rs);
        }
        l_run += rs;
        le_run += re;

        // O^T += V_j^T P^T: A operand = V^T rows 32dt + n, keys 16pc + 8hf + 0..7.
#pragma unroll
        for (int pc = 0; pc < PC; ++pc)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const int i = pc * DT + dt;
            const u32x4_t a =
                i < VPRE ? vpre[i < VPRE ? i : 0]
                         : *(const u32x4_t*)&vt_lds[buf][32 * dt + n][16 * pc + 8 * hf];
            acc[dt] = mfma_bf16(a, pb[pc], acc[dt]);
          }
        constexpr int VREST = PC * DT - VPRE;   // V^T operands read inside the P V loop
        mfma_read_ahead<PC * DT, (VREST < FA_READ_AHEAD ? VREST : FA_READ_AHEAD)>();
      }
      if (more) store_block(buf ^ 1);
      __syncthreads();
    }

    // Epilogue: O = acc / l (rounded to bf16 once), LSE = (m + log2 le) * ln 2.
    uint16_t* __restrict__ Oh =
        (uint16_t*)p.o + (GEN ? b * p.obs + hh * p.ohs + qr0 * p.ors : (long long)hoff);
    float* __restrict__ Lh = p.lse + (VL ? hh * p.total_q + qr0 : (long long)bh * N);
    const float lt = pair_sum(l_run);
    const float le = pair_sum(le_run);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int qrow = qw0 + n;
    if (qrow < N) {
      uint16_t* orow = Oh + (size_t)qrow * (GEN ? (size_t)p.ors : (size_t)D);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          u32x2_t x = {pack_bf16(acc[dt][4 * a] * inv, acc[dt][4 * a + 1] * inv),
                       pack_bf16(acc[dt][4 * a + 2] * inv, acc[dt][4 * a + 3] * inv)};
          *(u32x2_t*)(orow + 32 * dt + 8 * a + 4 * hf) = x;
        }
      if (hf == 0) Lh[qrow] = lt > 0.f ? (m_run + __builtin_amdgcn_logf(le)) * kLn2 : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16, d = 128, contiguous self-attention, scale > 0: 64 query rows per wave
// ---------------------------------------------------------------------------
// Four waves (one per SIMD), 256 query rows per work item.  Each K and V^T
// operand read from LDS feeds the MFMAs of two 32-row tiles, and the softmax
// of one key block runs beside the MFMAs of the neighbouring blocks inside
// one wave's instruction stream.  The block loop is one inline-asm program
// (fa_fwd_d128_loop.inc, written by gen_fwd_d128_loop.py, which documents the
// pipeline and the register plan); this function maps work items, computes
// the per-item scalars and lane offsets and hands them to it.
//
// LDS: three K slots, then three V slots, 20 KiB each.  K rows are 272 bytes
// apart and V rows 320, which makes the K operand reads (ds_read_b128) and
// the transposing V^T reads (ds_read_b64_tr_b16) free of bank conflicts.
// K and V blocks are staged with direct-to-LDS buffer loads: each wave
// instruction writes 1 KiB of the padded slot image in lane order, and each
// lane's source offset puts its 16 bytes where they belong (pad positions
// read past the buffer range and receive zeros).
constexpr int kD128Slot = 20480;
constexpr uint32_t kOutOfRange = 0x80000000u;

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void fa_fwd_d128_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[6 * kD128Slot];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int hf = lane >> 5;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;

  // Staging: instruction u of this wave fills bytes [1024 (wave + 4u), +1024)
  // of a slot.
  uint32_t ko[5], vo[5];
#pragma unroll
  for (int u = 0; u < 5; ++u) {
    const int pb = (wave + 4 * u) * 1024 + 16 * lane;
    const int kr = pb / 272, kc = pb % 272, vr = pb / 320, vc = pb % 320;
    ko[u] = (kr < 64 && kc < 256) ? (uint32_t)(kr * 256 + kc) : kOutOfRange;
    vo[u] = (vr < 64 && vc < 256) ? (uint32_t)(vr * 256 + vc) : kOutOfRange;
  }
  // K operand of S^T = K Q^T: row row_perm(n) of a 32-key tile, d 8hf..8hf+7
  // of each 16-wide step.  V^T operand: lanes 16g + j address V row
  // 8(g/2) + j/4 (+ 16 pc + 4 half), columns 16(g%2) + 4(j%4) (+ 32 dt); the
  // transposing read hands lane 16g + j the 4 keys of column 16(g%2) + j.
  const uint32_t kaddr = lds0 + (uint32_t)(row_perm(n) * 272 + 16 * hf);
  const int g = lane >> 4, j = lane & 15;
  const uint32_t vaddr =
      lds0 + 3 * kD128Slot + (uint32_t)((8 * (g >> 1) + (j >> 2)) * 320 + 32 * (g & 1) + 8 * (j & 3));
  const uint32_t ldsk = __builtin_amdgcn_readfirstlane(lds0 + 1024u * wave);
  const uint32_t ldsv = __builtin_amdgcn_readfirstlane(lds0 + 3 * kD128Slot + 1024u * wave);

  const bool causal = p.causal != 0;
  const int N = p.N;
  const int P = gridDim.x, G = p.items;
  const bool lanes8 = G % 8 == 0 && P % 8 == 0;
  const int L8 = lanes8 ? 8 : 1;
  const int lx = blockIdx.x % L8, mx = blockIdx.x / L8, Pm = P / L8, Gm = G / L8;
  for (int round = 0;; ++round) {
    const int idx = round * Pm + ((round & 1) ? Pm - 1 - mx : mx);
    if (idx >= Gm) break;
    int bh, qb;
    map_work(p.nqb, causal, p.hg, false, idx * L8 + lx, p.items, bh, qb);
    const int b = bh / p.H;
    const size_t hoff = (size_t)bh * (size_t)N * 128;
    const uint64_t qa = (uint64_t)((const uint16_t*)p.q + hoff);
    const uint64_t ka = (uint64_t)((const uint16_t*)p.k + hoff);
    const uint64_t va = (uint64_t)((const uint16_t*)p.v + hoff);
    const uint64_t oa = (uint64_t)((uint16_t*)p.o + hoff);
    const uint64_t la = (uint64_t)(p.lse + (size_t)bh * N);
    int n_vis = N;
    if (p.kv_lens) {
      const int kl = p.kv_lens[b];
      n_vis = kl < 0 ? 0 : (kl > N ? N : kl);
    }
    n_vis = __builtin_amdgcn_readfirstlane(n_vis);
    const int q0 = qb * 256;
    const int qw0 = q0 + 64 * wave;
    const int kend = causal ? min(n_vis, q0 + 256) : n_vis;
    const int nblk = __builtin_amdgcn_readfirstlane((kend + 63) / 64);
    // Last key block this wave visits (-1: none); only it can hold hidden keys.
    int jlast = -1;
    if (qw0 < N) {
      const int kv = causal ? min(n_vis, qw0 + 64) : n_vis;
      jlast = (kv + 63) / 64 - 1;
    }
    jlast = __builtin_amdgcn_readfirstlane(jlast);
    // Mask of that block: register index i (0..63) of a lane is hidden when
    // i > lim (key kb + i + 8hf against the lane's row).
    const int kb = 64 * (jlast > 0 ? jlast : 0);
    const int rowA = qw0 + n, rowB = qw0 + 32 + n;
    const int limA = (causal ? min(rowA, n_vis - 1) : n_vis - 1) - kb - 8 * hf;
    const int limB = (causal ? min(rowB, n_vis - 1) : n_vis - 1) - kb - 8 * hf;
    const uint32_t qoff0 = (uint32_t)rowA * 256u + 16u * hf, qoff1 = qoff0 + 8192u;
    const uint32_t ooff0 = (uint32_t)rowA * 256u + 8u * hf, ooff1 = ooff0 + 8192u;
    const uint32_t loff0 = hf ? kOutOfRange : (uint32_t)rowA * 4u;
    const uint32_t loff1 = hf ? kOutOfRange : (uint32_t)rowB * 4u;
    // K and V ranges end at the item's last key block: the staging of the
    // blocks after it (the loop stages two blocks ahead) reads out of range
    // and lands zeros without touching memory.
    const uint32_t nbytes = (uint32_t)N * 256u;
    const uint32_t kbytes = (uint32_t)min(N, 64 * nblk) * 256u;
    const uint32_t vbytes = (uint32_t)min(n_vis, 64 * nblk) * 256u;
    const uint32_t lbytes = (uint32_t)N * 4u;
#ifdef FA_D128_DEBUG
#ifdef FA_D128_PROFILE
    const uint32_t dbgoff = lane == 0 ? (uint32_t)((qb * 4 + wave) * 8 * 256) : kOutOfRange;
#else
    const uint32_t dbgoff = qb == 0 ? (uint32_t)(wave * 230 * 256 + lane * 4) : kOutOfRange;
#endif
#define FA_D128_DBG_OPERAND , [dbg] "v"(dbgoff)
#define FA_D128_BODY "fa_fwd_d128_loop_debug.inc"
#define FA_D128_CLOBBERS "fa_fwd_d128_clobbers_debug.inc"
#else
#define FA_D128_DBG_OPERAND
#define FA_D128_BODY "fa_fwd_d128_loop.inc"
#define FA_D128_CLOBBERS "fa_fwd_d128_clobbers.inc"
#endif
    asm volatile(
#include FA_D128_BODY
        :
        : [klo] "s"((uint32_t)ka), [khi] "s"((uint32_t)(ka >> 32)), [kbytes] "s"(kbytes),
          [vlo] "s"((uint32_t)va), [vhi] "s"((uint32_t)(va >> 32)), [vbytes] "s"(vbytes),
          [qlo] "s"((uint32_t)qa), [qhi] "s"((uint32_t)(qa >> 32)), [qbytes] "s"(nbytes),
          [olo] "s"((uint32_t)oa), [ohi] "s"((uint32_t)(oa >> 32)),
          [llo] "s"((uint32_t)la), [lhi] "s"((uint32_t)(la >> 32)), [lbytes] "s"(lbytes),
          [nblk] "s"(nblk), [jlast] "s"(jlast), [c] "s"(p.c), [ldsk] "s"(ldsk), [ldsv] "s"(ldsv),
          [ko0] "v"(ko[0]), [ko1] "v"(ko[1]), [ko2] "v"(ko[2]), [ko3] "v"(ko[3]),
          [ko4] "v"(ko[4]), [vo0] "v"(vo[0]), [vo1] "v"(vo[1]), [vo2] "v"(vo[2]),
          [vo3] "v"(vo[3]), [vo4] "v"(vo[4]), [qoff0] "v"(qoff0), [qoff1] "v"(qoff1),
          [ooff0] "v"(ooff0), [ooff1] "v"(ooff1), [loff0] "v"(loff0), [loff1] "v"(loff1),
          [kaddr] "v"(kaddr), [vaddr] "v"(vaddr), [limA] "v"(limA), [limB] "v"(limB)
          FA_D128_DBG_OPERAND
        :
#include FA_D128_CLOBBERS
    );
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
  map_work(p.nqb, causal, p.hg, bh, qb);
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

// Head dimensions of the bf16 forward kernels (the fp32 kernel: 64 and 128).
bool bf16_head_dim(int d) { return d == 32 || d == 64 || d == 96 || d == 128 || d == 256; }

int check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
               int B, int H, int N, int d, float scale, int mask_kind, const int32_t* kv_lens,
               int bm, int pad_rows, bool bf16) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  const uintptr_t al = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse;
  if (al & 15u) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
  if (mask_kind & ~(FA_MASK_CAUSAL | FA_MASK_KEY_PADDING)) return FA_ERR_INVALID_ARG;
  if ((mask_kind & FA_MASK_KEY_PADDING) && !kv_lens) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (bf16 ? !bf16_head_dim(d) : (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
  const long long nqb = ((long long)N + bm - 1) / bm;
  if ((long long)B * H * nqb > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  // One head's rows (plus pad_rows past the end) are addressed with 32-bit
  // byte offsets.
  if (((long long)N + pad_rows) * d * 4 > 0xffffffffLL) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

Params make_params(const void* q, const void* k, const void* v, void* o, float* lse, int H, int N,
                   int nqb, float scale, int mask_kind, const int32_t* kv_lens) {
  Params p = {};
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
  p.hg = 4;
  return p;
}

// One bf16 forward launch over p.items work items.  Contiguous
// self-attention with d <= 128 launches at most as many workgroups as the
// chip holds at once and lets each loop over its items (no workgroup start
// per item; the snake order of the kernel balances the causal ranks); the
// other layouts and d = 256 launch one workgroup per item.
template <int D, int NW, int MODE>
void launch_one(hipStream_t s, Params p) {
  static std::atomic<long long> cache{0};
  const long long resident = resident_workgroups(fa_fwd_bf16_kernel<D, NW, MODE>, 64 * NW, cache);
  p.hg = head_group(p.causal != 0, p.items, resident);
  const long long cap = resident > 0 ? resident : kCUs;
  const long long grid = (MODE == 0 && D <= 128) ? std::min<long long>(p.items, cap) : p.items;
  hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, NW, MODE>), dim3((unsigned)grid), dim3(64 * NW), 0,
                     s, p);
}

// The 64-rows-per-wave d = 128 kernel: at most as many workgroups as the chip
// holds (one per CU), each looping over 256-row items in snake order.
void launch_d128(hipStream_t s, Params p) {
  static std::atomic<long long> cache{0};
  const long long resident = resident_workgroups(fa_fwd_d128_kernel, 256, cache);
  p.hg = head_group(p.causal != 0, p.items, resident);
  const long long cap = resident > 0 ? resident : kCUs;
  const long long grid = std::min<long long>(p.items, cap);
  hipLaunchKernelGGL(fa_fwd_d128_kernel, dim3((unsigned)grid), dim3(256), 0, s, p);
}

// FA92_FWD_D128=0 in the environment sends d = 128 to the 32-rows-per-wave
// kernel as well (read once per process; for side-by-side comparisons).
bool use_d128_kernel() {
  static const int on = [] {
    const char* e = getenv("FA92_FWD_D128");
    return (e && e[0] == '0') ? 0 : 1;
  }();
  return on != 0;
}

// 8-wave (256-row) workgroups when big, else 4-wave.
template <int MODE>
void launch_bf16(int d, bool big, hipStream_t s, const Params& p) {
#define FA_LAUNCH(DD)                      \
  if (big) launch_one<DD, 8, MODE>(s, p);  \
  else launch_one<DD, 4, MODE>(s, p)
  switch (d) {
    case 32: FA_LAUNCH(32); break;
    case 64: FA_LAUNCH(64); break;
    case 96: FA_LAUNCH(96); break;
    case 128: FA_LAUNCH(128); break;
    default:   // 256: 4-wave (128-row) workgroups only, one wave per SIMD
      launch_one<256, 4, MODE>(s, p);
      break;
  }
#undef FA_LAUNCH
}

}  // namespace

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int N, int d, float scale, int mask_kind, const int32_t* kv_lens,
                      void* stream) {
  // Work items are 128- or 256-row query blocks: B * H * ceil(N / 128)
  // bounds both grids.
  const int st =
      check_args(q, k, v, o, lse, B, H, N, d, scale, mask_kind, kv_lens, 128, 256, true);
  if (st != FA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (d == 128 && scale > 0.f && use_d128_kernel()) {
    const int nqb = (N + 255) / 256;
    Params p = make_params(q, k, v, o, lse, H, N, nqb, scale, mask_kind, kv_lens);
    p.items = B * H * nqb;
    launch_d128(s, p);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
  }
  // 256-row workgroups (8 waves, one per CU) share each K/V tile among more
  // rows.  They are used when they fill the 256 CUs at least once (twice for
  // causal masks, whose query blocks differ in cost); otherwise 128-row
  // workgroups (two per CU) balance better.
  const long long grid256 = (long long)B * H * ((N + 255) / 256);
  const bool big = d != 256 && grid256 >= ((mask_kind & FA_MASK_CAUSAL) ? 2 : 1) * kCUs;
  const int BM = big ? 256 : 128;
  const int nqb = (N + BM - 1) / BM;
  Params p = make_params(q, k, v, o, lse, H, N, nqb, scale, mask_kind, kv_lens);
  p.items = B * H * nqb;
  launch_bf16<0>(d, big, s, p);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_fwd_general(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int Nq, int Nk, int d, const int64_t* q_strides,
                              const int64_t* k_strides, const int64_t* v_strides,
                              const int64_t* o_strides, float scale, int mask_kind,
                              int window_left, const int32_t* kv_lens, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  const uintptr_t al = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse;
  if (al & 15u) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || window_left < -1) return FA_ERR_INVALID_ARG;
  if (mask_kind & ~(FA_MASK_CAUSAL | FA_MASK_KEY_PADDING)) return FA_ERR_INVALID_ARG;
  if ((mask_kind & FA_MASK_KEY_PADDING) && !kv_lens) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (!bf16_head_dim(d)) return FA_ERR_UNSUPPORTED;
  // Strides (elements): NULL = contiguous [B, H, rows, d].  Rows must be
  // 16-byte aligned and hold d contiguous elements; batch and head starts
  // 16-byte aligned.
  int64_t st[4][3];
  const int64_t* given[4] = {q_strides, k_strides, v_strides, o_strides};
  const int rows[4] = {Nq, Nk, Nk, Nq};
  for (int t = 0; t < 4; ++t) {
    if (given[t]) {
      for (int i = 0; i < 3; ++i) st[t][i] = given[t][i];
    } else {
      st[t][2] = d;
      st[t][1] = (int64_t)rows[t] * d;
      st[t][0] = (int64_t)H * rows[t] * d;
    }
    if (st[t][2] < d || st[t][0] < 0 || st[t][1] < 0) return FA_ERR_INVALID_ARG;
    if ((st[t][0] | st[t][1] | st[t][2]) & 7) return FA_ERR_INVALID_ARG;
    // A head's rows (plus a block past the end) use 32-bit byte offsets.
    if (((long long)rows[t] + 256) * st[t][2] * 2 > 0xffffffffLL) return FA_ERR_INVALID_ARG;
  }
  const bool causal = (mask_kind & FA_MASK_CAUSAL) != 0;
  const long long grid256 = (long long)B * H * ((Nq + 255) / 256);
  const bool big = d != 256 && grid256 >= (causal ? 2 : 1) * kCUs;
  const int BM = big ? 256 : 128;
  const int nqb = (Nq + BM - 1) / BM;
  if ((long long)B * H * nqb > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  Params p = make_params(q, k, v, o, lse, H, Nq, nqb, scale, mask_kind, kv_lens);
  p.Nk = Nk;
  p.off = Nk - Nq;
  p.window = window_left;
  p.qbs = st[0][0]; p.qhs = st[0][1]; p.qrs = (unsigned)(st[0][2] * 2);
  p.kbs = st[1][0]; p.khs = st[1][1]; p.krs = (unsigned)(st[1][2] * 2);
  p.vbs = st[2][0]; p.vhs = st[2][1]; p.vrs = (unsigned)(st[2][2] * 2);
  p.obs = st[3][0]; p.ohs = st[3][1]; p.ors = (unsigned)st[3][2];
  p.items = B * H * nqb;
  launch_bf16<1>(d, big, (hipStream_t)stream, p);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                             int H, int d, int64_t total_q, int64_t total_k, int max_seqlen_q,
                             float scale, int mask_kind, int window_left, void* stream) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_INVALID_ARG;
  const uintptr_t al = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse;
  if (al & 15u) return FA_ERR_INVALID_ARG;
  if (((uintptr_t)cu_seqlens_q | (uintptr_t)cu_seqlens_k) & 3u) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || window_left < -1)
    return FA_ERR_INVALID_ARG;
  if (mask_kind & ~FA_MASK_CAUSAL) return FA_ERR_INVALID_ARG;   // lengths come from cu_seqlens_k
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (!bf16_head_dim(d)) return FA_ERR_UNSUPPORTED;
  if (max_seqlen_q == 0 || total_q == 0) return FA_OK;          // no query rows: nothing to write
  if (max_seqlen_q > total_q) max_seqlen_q = (int)total_q;
  // Packed rows are H*d elements apart; a sequence's rows (plus a block past
  // the end) use 32-bit byte offsets.
  const long long rowb = (long long)H * d * 2;
  if ((total_q + 256) * rowb > 0xffffffffLL || (total_k + 256) * rowb > 0xffffffffLL)
    return FA_ERR_INVALID_ARG;
  const bool causal = (mask_kind & FA_MASK_CAUSAL) != 0;
  const long long grid256 = (long long)B * H * ((max_seqlen_q + 255) / 256);
  const bool big = d != 256 && grid256 >= (causal ? 2 : 1) * kCUs;
  const int BM = big ? 256 : 128;
  const int nqb = (max_seqlen_q + BM - 1) / BM;
  if ((long long)B * H * nqb > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  Params p = make_params(q, k, v, o, lse, H, max_seqlen_q, nqb, scale, mask_kind, nullptr);
  p.window = window_left;
  p.qhs = d; p.qrs = (unsigned)rowb;
  p.khs = d; p.krs = (unsigned)rowb;
  p.vhs = d; p.vrs = (unsigned)rowb;
  p.ohs = d; p.ors = (unsigned)(H * d);
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.total_q = total_q;
  p.total_k = total_k;
  p.items = B * H * nqb;
  launch_bf16<2>(d, big, (hipStream_t)stream, p);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                          int H, int N, int d, float scale, int mask_kind, const int32_t* kv_lens,
                          void* stream) {
  constexpr int BM = 32 * kWaves;
  const int st = check_args(q, k, v, o, lse, B, H, N, d, scale, mask_kind, kv_lens, BM, BM, false);
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
    case FA_ERR_UNSUPPORTED:
      return "unsupported head dimension (bf16 forward: 32, 64, 96, 128, 256; others: 64, 128)";
    case FA_ERR_HIP: return "HIP launch failure";
    case FA_ERR_SCRATCH:
      return "the call needs more scratch than the fixed buffer of the no-allocation entry point";
    default: return "unknown status";
  }
}
