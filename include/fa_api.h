/*
 * fa_api.h -- C ABI of the exact attention library (libfa92.so): the
 * forward pass (bf16, fp32, fp8), the backward pass and paged decode.
 *
 * What the library computes, for every batch entry b and head h:
 *
 *     O   = softmax(scale * Q K^T + M) V
 *     LSE = m + ln(l)        (per query row: row max m and row sum l of the
 *                             exponentials of the scaled, masked logits)
 *
 * This is the exact scaled-dot-product attention of "FlashAttention算法详解：
 * 从IO瓶颈到Triton实现" (gentlecold.top), section 先说结论 (the equation), with
 * LSE as in its section Backward为什么更复杂.  It is computed IO-aware: each
 * block of query rows streams over blocks of keys and values with the
 * online-softmax state (running max, running sum, rescaled accumulator) of
 * that page's sections Online Softmax and FlashAttention Forward流程, so the
 * N x N scores and probabilities never reach device memory.
 *
 * Conventions shared by both entry points:
 *
 *  - q, k, v, o: DEVICE pointers to contiguous row-major tensors of shape
 *    [B, H, N, d] (batch, head, sequence, head dimension).  Element type is
 *    bfloat16 for fa_fwd and float32 for fa_fwd_f32; o has the input type.
 *    Every pointer must be 16-byte aligned.  Self-attention: queries and keys
 *    share the length N.
 *  - lse: DEVICE pointer to float32 [B, H, N], natural-log units of the
 *    scaled logits.  A query row with no visible key gets O = 0 and
 *    LSE = -inf.
 *  - B, H, N >= 1; d is 32, 64, 96, 128 or 256 for fa_fwd, 64 or 128 for
 *    fa_fwd_f32.  B * H * ceil(N / 128) must not exceed 2^31 - 1, and
 *    (N + 256) * d * 4 (fa_fwd; N + 128 for fa_fwd_f32) must not exceed
 *    2^32 - 1: one head's rows, plus one block past the end, are addressed
 *    with 32-bit byte offsets.  So N <= 16776959 at d = 64 and 8388351 at
 *    d = 128 for fa_fwd.
 *  - scale: any finite float; the logits are scale * q.k.  (1/sqrt(d) is the
 *    usual value.)  |scale| below 1e-30 is treated as 1e-30, which gives the
 *    same uniform softmax as scale = 0 to within float32 rounding.
 *  - mask_kind: bit flags.  FA_MASK_CAUSAL hides key c from query r when
 *    c > r (the diagonal stays visible; "Causal Mask怎么处理" on the page
 *    above).  FA_MASK_KEY_PADDING hides keys c >= kv_lens[b] from every
 *    query row and head of batch entry b.  Both flags: the union of the
 *    hidden sets.  Other bits are rejected.
 *  - kv_lens: DEVICE pointer to int32 [B], required when FA_MASK_KEY_PADDING
 *    is set, ignored (may be NULL) otherwise.  Values are read on the device
 *    and clamped to [0, N].
 *  - stream: a hipStream_t (NULL = the default stream).  The call enqueues
 *    one kernel on it and returns without synchronising.
 *
 * Ownership and side effects: the caller owns every buffer; the library
 * allocates no memory.  Its only state is a process-wide cache of how many
 * workgroups of each kernel the device holds at once (the first occupancy
 * query that succeeds; it sets the grid size and the order of the work
 * only).  It writes o and lse and nothing else.  Inputs are only
 * read.
 *
 * Errors: every argument is checked on the host before anything is
 * enqueued; on an error the call returns a negative status and writes
 * nothing.  FA_ERR_HIP reports a launch failure (from hipGetLastError).
 * Faults that happen while the kernel runs surface at the caller's next
 * synchronisation, as with any asynchronous launch.
 */
#ifndef FA_API_H
#define FA_API_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  FA_MASK_NONE = 0,
  FA_MASK_CAUSAL = 1,
  FA_MASK_KEY_PADDING = 2
};

enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size, bad mask bits,
                              non-finite scale, padding without kv_lens */
  FA_ERR_UNSUPPORTED = -2, /* head dimension the entry point does not support */
  FA_ERR_HIP = -3,         /* the kernel launch failed */
  FA_ERR_SCRATCH = -4      /* needs more scratch than the no-allocation entry
                              point's fixed buffer holds */
};

/* bfloat16 forward.  q, k, v, o: bf16 [B, H, N, d]; lse: float32 [B, H, N].
 * Products run on the bf16 matrix cores with float32 accumulation; the
 * probabilities are rounded to bf16 before they multiply V (as the pages'
 * Triton sketch does with p.to(v.dtype)); O is rounded to bf16 (nearest,
 * ties to even) once, at the end. */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int mask_kind,
           const int32_t* kv_lens, void* stream);

/* float32 forward: same contract with float32 q, k, v, o.  Every product and
 * sum is float32 (matrix-core fp32 multiply-accumulate); nothing is rounded
 * to a narrower type. */
int fa_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int mask_kind,
               const int32_t* kv_lens, void* stream);

/* General bf16 forward: fa_fwd with separate query and key counts, a
 * sliding window and arbitrary strides (the variants of the forward that
 * "FlashAttention 完整解析" §11 and the youngju.dev walkthrough §11 list
 * for the library: cross-attention lengths, local windows, layouts).
 *  - q, o: [B, H, Nq, d]; k, v: [B, H, Nk, d], each addressed through its
 *    own strides: HOST int64 arrays {batch, head, row} in elements (NULL:
 *    contiguous).  Rows hold d contiguous elements; every stride is a
 *    multiple of 8 elements (16 bytes) and the row stride at least d, so
 *    e.g. the [B, N, H, d] layout is strides {N*H*d, d, H*d}.  lse is a
 *    contiguous float32 [B, H, Nq].
 *  - Query row r sits at key position a_r = r + Nk - Nq (the queries are the
 *    last Nq positions of the key sequence).  Key c is visible to row r iff
 *    c < kv_len (key padding), c <= a_r (FA_MASK_CAUSAL), and
 *    c >= a_r - window_left when window_left >= 0 (window_left = -1: no
 *    window).  A row that sees no key gets O = 0, LSE = -inf.
 *  - Nq, Nk >= 1; d is 32, 64, 96, 128 or 256; 16-byte aligned pointers.
 *    B * H * ceil(Nq / 128) must not exceed 2^31 - 1, and for each tensor
 *    (rows + 256) * row_stride * 2 must not exceed 2^32 - 1 (rows = Nq for
 *    q and o, Nk for k and v): a head's rows use 32-bit byte offsets.  Other
 *    conventions (scale, kv_lens, stream, errors) as for fa_fwd.  With
 *    contiguous strides, Nq = Nk and no window it computes exactly fa_fwd. */
int fa_fwd_general(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Nq, int Nk, int d, const int64_t* q_strides,
                   const int64_t* k_strides, const int64_t* v_strides,
                   const int64_t* o_strides, float scale, int mask_kind, int window_left,
                   const int32_t* kv_lens, void* stream);

/* Variable-length bf16 forward over packed sequences (the variable-length
 * batches that "FlashAttention 完整解析" §11 lists for the library): B
 * sequences of different lengths stored back to back, each attended on its
 * own exactly as fa_fwd_general attends one batch entry.
 *  - q, o: DEVICE bf16 [total_q, H, d]; k, v: DEVICE bf16 [total_k, H, d],
 *    contiguous, 16-byte aligned.  lse: DEVICE float32 [H, total_q].
 *  - cu_seqlens_q, cu_seqlens_k: DEVICE int32 [B + 1], non-decreasing,
 *    starting at 0: sequence b owns query rows cu_seqlens_q[b] ..
 *    cu_seqlens_q[b+1] - 1 and key rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]
 *    - 1.  Its Nq_b queries sit at the last Nq_b of its Nk_b key positions;
 *    causal and window_left act as in fa_fwd_general within the sequence.
 *    The values are not read on the host: each is clamped into [0, total]
 *    on the device, so bad values cannot reach outside the tensors (the
 *    result is then meaningless, and overlapping sequences race).
 *  - max_seqlen_q must be at least every Nq_b: rows past it are not
 *    written.  mask_kind: FA_MASK_NONE or FA_MASK_CAUSAL (key lengths come
 *    from cu_seqlens_k).  A sequence with Nk_b = 0 gets O = 0, LSE = -inf.
 *  - total_q = 0 or max_seqlen_q = 0 enqueues nothing.  (total_q + 256) *
 *    H * d * 2 and (total_k + 256) * H * d * 2 must not exceed 2^32 - 1.
 *    Other conventions (d, scale, stream, errors) as for fa_fwd_general. */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int H,
                  int d, int64_t total_q, int64_t total_k, int max_seqlen_q, float scale,
                  int mask_kind, int window_left, void* stream);

/* FP8 forward (the FP8 path of "FlashAttention 完整解析" §5.5 and of the
 * youngju.dev walkthrough §9.2): q, k, v hold OCP FP8 E4M3 codes
 * ("e4m3fn": bias 7, largest finite 448, no infinities) of shape
 * [B, H, N, d]; each (batch, head) has one float32 scale per tensor, so the
 * values are q_code * q_descale[b*H + h] and likewise for k and v (block
 * quantization with one block per head).  The result is the attention of
 * those values, with the same mask, scale, LSE and empty-row conventions as
 * fa_fwd; o is bfloat16 [B, H, N, d], lse float32 [B, H, N].
 *  - Products run on the E4M3 matrix cores with float32 accumulation.  The
 *    probabilities are taken against a reference max that lags the row max
 *    by at most 2 binary orders (so each is at most 4), multiplied by 448/4
 *    and rounded to E4M3 before they multiply V; the factor cancels in the
 *    normalisation, which divides by the float32 sum of the unrounded
 *    values.  Rounding P to E4M3 (relative error up to 2^-4) is the
 *    dominant error of this path.
 *  - q_descale, k_descale, v_descale: DEVICE pointers to float32 [B * H],
 *    4-byte aligned, finite and positive (not checked on the host).
 *  - Everything else as for fa_fwd. */
int fa_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale,
               const float* k_descale, const float* v_descale, void* o, float* lse,
               int B, int H, int N, int d, float scale, int mask_kind,
               const int32_t* kv_lens, void* stream);

/* Rows per scale tile of fa_fwd_fp8_tiled. */
#define FA_FP8_TILE 128

/* FP8 forward with block quantization at tile granularity (the youngju.dev
 * walkthrough §9.2, "block quantization": an independent scale per block to
 * keep the dynamic range; "FlashAttention 完整解析" §5.5, scaling per tile
 * before the softmax): as fa_fwd_fp8, except that Q and K carry one float32
 * scale per FA_FP8_TILE consecutive rows of each head, so the values are
 * q_code[b,h,r,:] * q_descale[(b*H + h)*T + r/FA_FP8_TILE] and likewise for
 * k, with T = ceil(N / FA_FP8_TILE).  Each (query tile, key tile) block of
 * the logits is a product of E4M3 codes times q_scale * k_scale * scale,
 * applied to the fp32 MFMA result before the softmax.  V keeps one scale per
 * (batch, head): v_descale[b*H + h].
 *  - q_descale, k_descale: DEVICE pointers to float32 [B * H * T];
 *    v_descale: float32 [B * H]; 4-byte aligned, finite and positive (not
 *    checked on the host).
 *  - Everything else (layouts, masks, bounds, precision, errors) as for
 *    fa_fwd_fp8. */
int fa_fwd_fp8_tiled(const void* q, const void* k, const void* v, const float* q_descale,
                     const float* k_descale, const float* v_descale, void* o, float* lse,
                     int B, int H, int N, int d, float scale, int mask_kind,
                     const int32_t* kv_lens, void* stream);

/* Decode over a paged KV cache ("FlashAttention 完整解析" §7, PageAttention's
 * block table): for each request b and head h, the one query vector
 * q[b, h, :] attends to the request's n_b = seq_lens[b] cached tokens,
 * which are stored in a pool of fixed-size blocks:
 *
 *     k_t = k_pool[block_tables[b, t / block_size], h, t % block_size, :]
 *     O[b, h] = softmax(scale * q . k_t over t < n_b) V,   LSE[b, h]
 *
 * (v_t likewise), i.e. the newest token's row of causal attention.
 *  - q: DEVICE bf16 [B, H, d]; k_pool, v_pool: DEVICE bf16
 *    [num_blocks, H, block_size, d]; all 16-byte aligned, read only.
 *  - block_tables: DEVICE int32 [B, max_blocks_per_seq]; entries past a
 *    request's last block are never read; an entry outside [0, num_blocks)
 *    reads as zeros (memory-safe; the result is then meaningless).
 *  - seq_lens: DEVICE int32 [B], clamped on the device to
 *    [0, max_blocks_per_seq * block_size]; n_b = 0 gives O = 0, LSE = -inf.
 *  - o: DEVICE bf16 [B, H, d]; lse: DEVICE float32 [B, H].
 *  - workspace: DEVICE float32 scratch of fa_decode_paged_workspace_bytes()
 *    bytes, caller-owned; it holds per-chunk partial results between the two
 *    kernels the call enqueues (calls that share a workspace must not
 *    overlap).
 *  - d is 64 or 128; block_size a multiple of 8 (8 .. 65536); any finite
 *    scale; B, H <= 65535; block_size * max_blocks_per_seq <= 2^31 - 1.
 *    Errors as for fa_fwd.  The library allocates
 *    nothing. */
size_t fa_decode_paged_workspace_bytes(int B, int H, int d, int block_size,
                                       int max_blocks_per_seq);
int fa_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_tables, const int32_t* seq_lens, void* o,
                    float* lse, float* workspace, int B, int H, int d, int block_size,
                    int max_blocks_per_seq, int num_blocks, float scale, void* stream);

/* The same decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no workspace argument; the per-chunk partial results live in a
 * fixed-size buffer the library holds in each GPU's memory (a file-scope
 * device array of FA_DECODE_NOALLOC_SCRATCH_BYTES, looked up once per
 * device on the first call made with that device current).  The call
 * allocates nothing.
 *  - Arguments as for fa_decode_paged, without workspace.
 *  - Returns FA_ERR_SCRATCH (and enqueues nothing) when
 *    fa_decode_paged_workspace_bytes() of the same sizes exceeds
 *    FA_DECODE_NOALLOC_SCRATCH_BYTES (16 MiB; B = 32, H = 32, d = 128 with
 *    8192 cached tokens per request needs 8.5 MB).
 *  - Every call on one GPU uses that GPU's single buffer: calls that may
 *    run at the same time on one GPU (different streams, or overlapping
 *    graph launches) race and must not be issued.  Nothing in the buffer
 *    needs to start at zero; it keeps the last call's partial results. */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES (16u << 20)
int fa_decode_paged_noalloc(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_tables, const int32_t* seq_lens, void* o,
                            float* lse, int B, int H, int d, int block_size,
                            int max_blocks_per_seq, int num_blocks, float scale, void* stream);

/* bfloat16 backward: the gradients of the attention above with respect to
 * q, k and v, given the upstream gradient dout = dL/dO.  With P the softmax
 * probabilities of the forward ("FlashAttention算法详解：从IO瓶颈到Triton实现",
 * section Backward为什么更复杂, with the scale carried by the scores):
 *
 *     dv = P^T dout
 *     dP = dout v^T,   dS = P * (dP - rowsum(dP * P))   (elementwise)
 *     dq = scale * dS k,   dk = scale * dS^T q
 *
 * P is rebuilt block by block from q, k and the forward's lse, so o and lse
 * must be the outputs of fa_fwd on the same q, k, v, scale, mask_kind and
 * kv_lens.  rowsum(dP * P) is computed as rowsum(dout * o), which is equal
 * since O = P V.
 *
 *  - q, k, v, o, dout: DEVICE pointers, bf16 [B, H, N, d], read only.
 *  - lse: DEVICE pointer, float32 [B, H, N], read only.
 *  - dq, dk, dv: DEVICE pointers, bf16 [B, H, N, d], written (every element;
 *    keys that no query sees get dk = dv = 0, a query that sees no key gets
 *    dq = 0).  Rounded to bf16 once, at the end.
 *  - dp_rowsum: DEVICE pointer, float32 [B, H, N], written with
 *    rowsum(dP * P) of every query row; the call also reads it back, so it
 *    is caller-owned scratch that must not alias any other argument.
 *  - Output buffers must not overlap each other or the inputs.
 *  - Sizes, scale, mask_kind, kv_lens, alignment, stream and errors: as for
 *    fa_fwd.  The call enqueues two kernels on the stream (dq and
 *    dp_rowsum, then dk and dv) and returns without synchronising; it
 *    allocates nothing and uses no atomics, so results are bitwise
 *    reproducible. */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout, void* dq, void* dk, void* dv,
           float* dp_rowsum, int B, int H, int N, int d, float scale,
           int mask_kind, const int32_t* kv_lens, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_API_H */
