// Device helpers shared by the attention kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace fa92 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMinScale = 1e-30f;

// D = A B + C on a 32x32 tile with a 16-deep bf16 contraction.  Lane l
// supplies A row l%32 and B column l%32, elements 8(l/32)..8(l/32)+7 of the
// contraction; it receives column l%32 of C, rows 8(r/4) + 4(l/32) + r%4 in
// register r.
__device__ __forceinline__ f32x16_t mfma_bf16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// Lane l's value combined with lane (l ^ 32)'s.
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max(lane l's value, lane (l ^ 32)'s value).
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Two floats -> packed bf16 pair (round to nearest even).
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2_t));
}

// acc + a.lo*b.lo + a.hi*b.hi over packed bf16 pairs, in fp32.
__device__ __forceinline__ float dot_bf16x2(unsigned a, unsigned b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// acc + (lo + hi) of a packed bf16 pair, in fp32.
__device__ __forceinline__ float sum_bf16x2(unsigned pair, float acc) {
  return dot_bf16x2(pair, 0x3f803f80u, acc);
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
// Word 3 selects the raw 32-bit data format used by CDNA buffer loads.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load16(rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
}

// Operand row that MFMA row m reads: bits 2 and 3 of m swapped.  With it,
// accumulator register r of lane-half h holds logical row 16*(r/8) + 8*h +
// (r%8) of each 32-row tile, so 8 consecutive registers are 8 consecutive
// rows: rounded to bf16 they are directly an MFMA operand whose contraction
// runs over those rows.
__device__ __forceinline__ int row_perm(int m) {
  return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Four 16-byte row pieces (rows i = 0..3, 8 bf16 each) -> the same data
// transposed: for each of the 8 columns, the 4 rows' values packed in 8
// bytes.  out_lo[w] holds column 2w, out_hi[w] column 2w+1.
__device__ __forceinline__ void transpose4x8(const u32x4_t (&x)[4], u32x2_t (&out_lo)[4],
                                             u32x2_t (&out_hi)[4]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const unsigned a0 = x[0][w], a1 = x[1][w], a2 = x[2][w], a3 = x[3][w];
    out_lo[w] = u32x2_t{__builtin_amdgcn_perm(a1, a0, 0x05040100u),
                        __builtin_amdgcn_perm(a3, a2, 0x05040100u)};
    out_hi[w] = u32x2_t{__builtin_amdgcn_perm(a1, a0, 0x07060302u),
                        __builtin_amdgcn_perm(a3, a2, 0x07060302u)};
  }
}

// Workgroups are dispatched round-robin over the 8 XCDs (w % 8), in order
// within one.  Maps work item w of G (nb blocks for each of G / nb heads) to
// (head bh, block blk).  When the heads split evenly, XCD x owns the heads
// bh = x, x + 8, x + 16, ... (each head's tensors stay in one XCD's L2, and
// every XCD gets heads of every batch entry, so per-batch key lengths
// balance across XCDs) and visits their blocks rank by rank, hg heads at a
// time (head_group below); rank 0 is block nb-1 when heavy_last (causal
// query blocks: heaviest first), else block 0.  Otherwise XCD x gets the
// contiguous logical range [x*G/8, (x+1)*G/8).  With spread (packed
// sequences of unequal lengths, where binding heads to XCDs would bind
// whole sequences to them) the order is rank-major over all heads.
__device__ __forceinline__ void map_work(int nb, bool heavy_last, int hg, bool spread, int w,
                                         int G, int& bh, int& blk) {
  const int BH = G / nb;
  if (spread) {
    bh = w % BH;
    const int r = w / BH;
    blk = heavy_last ? (nb - 1 - r) : r;
    return;
  }
  if (G % 8 == 0 && BH % 8 == 0) {
    const int hx = BH / 8, i = w / 8;
    const int g = (hx % hg == 0) ? hg : hx;
    const int grp = i / (g * nb), j = i - grp * (g * nb);
    bh = (grp * g + j % g) * 8 + (w % 8);
    const int r = j / g;
    blk = heavy_last ? (nb - 1 - r) : r;
    return;
  }
  const int L = (G % 8 == 0) ? (w % 8) * (G / 8) + w / 8 : w;
  bh = L / nb;
  const int r = L - bh * nb;
  blk = heavy_last ? (nb - 1 - r) : r;
}

// The same for a launch with one workgroup per work item.
__device__ __forceinline__ void map_work(int nb, bool heavy_last, int hg, int& bh, int& blk) {
  map_work(nb, heavy_last, hg, false, (int)blockIdx.x, (int)gridDim.x, bh, blk);
}

// Compute units of an MI355X: the grid size of a looping launch while the
// runtime cannot say how many workgroups the chip holds.
constexpr long long kCUs = 256;

// Workgroups of `kernel` the device holds at once (occupancy per compute
// unit x compute units), cached in `cache` once a query succeeds; 0 while
// the runtime cannot answer (nothing is cached then, and the failed query
// is not left as the caller's error).
template <typename Kernel>
inline long long resident_workgroups(Kernel kernel, int threads, std::atomic<long long>& cache) {
  const long long known = cache.load(std::memory_order_relaxed);
  if (known > 0) return known;
  int occ = 0, dev = 0, cus = 0;
  const bool ok =
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, 0) == hipSuccess &&
      occ > 0 && hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      cus > 0;
  (void)hipGetLastError();
  if (!ok) return 0;
  cache.store((long long)occ * cus, std::memory_order_relaxed);
  return (long long)occ * cus;
}

// Heads per map_work group: 8 for causal launches whose work items are all
// resident at once (known resident count) -- each CU then holds items a
// fixed distance apart in its XCD's order, and a rank-major run over 8 heads
// puts a heavy causal rank and a light one there where a run over 4 pairs
// equal ranks -- else 4, which keeps the L2 working set smaller.
inline int head_group(bool causal, long long items, long long resident) {
  return (causal && resident > 0 && items <= resident) ? 8 : 4;
}

}  // namespace fa92
