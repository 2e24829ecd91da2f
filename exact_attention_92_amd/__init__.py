"""Exact attention on MI355X (gfx950): Python binding of libfa92.so.

The binding only marshals arguments: every step of the forward and backward
passes runs in the HIP kernels of ``csrc/fa_fwd.hip``, ``csrc/fa_fwd_fp8.hip``,
``csrc/fa_bwd_kernels.h`` and ``csrc/fa_decode.hip``.  PyTorch supplies device memory and
the stream.  There is no CPU or PyTorch fallback: if the library is missing
or the GPU is absent, the calls raise.

Names follow the C ABI of ``include/fa_api.h``:

* ``fa_fwd(q, k, v, o, lse, scale, mask_kind=0, kv_lens=None, stream=None)``
  -- bf16 tensors ``[B, H, N, d]``
* ``fa_fwd_f32(...)`` -- the same with float32 tensors
* ``fa_fwd_general(q, k, v, o, lse, scale, mask_kind=0, window_left=-1,
  kv_lens=None, stream=None)`` -- bf16 with Nq != Nk, a sliding window and
  any tensor strides (q, o [B, H, Nq, d] and k, v [B, H, Nk, d] views)
* ``fa_fwd_fp8(q, k, v, q_descale, k_descale, v_descale, o, lse, scale,
  mask_kind=0, kv_lens=None, stream=None)`` -- E4M3 codes (uint8 tensors)
  with per-(batch, head) float32 scales; o is bf16
* ``fa_fwd_fp8_tiled(...)`` -- the same with one q / k scale per 128 rows
  (``q_descale``, ``k_descale`` float32 ``[B, H, ceil(N / 128)]``)
* ``fa_decode_paged(q, k_pool, v_pool, block_tables, seq_lens, o, lse,
  workspace, scale, stream=None)`` and
  ``fa_decode_paged_workspace_bytes(B, H, d, block_size, max_blocks)``
* ``fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, dp_rowsum, scale, mask_kind=0,
  kv_lens=None, stream=None)`` -- bf16 gradients
* ``fa_strerror(status)``

``attention(q, k, v, ...)`` allocates ``o`` and ``lse`` and calls the right
entry point.
"""
from __future__ import annotations

import ctypes
import os

FA_MASK_NONE = 0
FA_MASK_CAUSAL = 1
FA_MASK_KEY_PADDING = 2

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_HIP = -3
FA_ERR_SCRATCH = -4
DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa92.so")
EXPORTS = ("fa_fwd", "fa_fwd_f32", "fa_fwd_general", "fa_fwd_varlen", "fa_fwd_fp8",
           "fa_fwd_fp8_tiled", "fa_bwd",
           "fa_decode_paged", "fa_decode_paged_noalloc", "fa_decode_paged_workspace_bytes",
           "fa_strerror")

_lib = None


class FaError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def load_library():
    """Load libfa92.so (built in-tree) and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run exact_attention_92_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    for name in ("fa_fwd", "fa_fwd_f32"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, vp]
        fn.restype = i32
    lib.fa_fwd_general.argtypes = [vp] * 5 + [i32] * 5 + [vp] * 4 + [f32, i32, i32, vp, vp]
    lib.fa_fwd_general.restype = i32
    lib.fa_fwd_varlen.argtypes = [vp] * 7 + [i32] * 3 + [ctypes.c_int64] * 2 + [i32, f32, i32,
                                                                               i32, vp]
    lib.fa_fwd_varlen.restype = i32
    for name in ("fa_fwd_fp8", "fa_fwd_fp8_tiled"):
        fn = getattr(lib, name)
        fn.argtypes = [vp] * 8 + [i32, i32, i32, i32, f32, i32, vp, vp]
        fn.restype = i32
    lib.fa_decode_paged.argtypes = [vp] * 8 + [i32] * 6 + [f32, vp]
    lib.fa_decode_paged.restype = i32
    lib.fa_decode_paged_noalloc.argtypes = [vp] * 7 + [i32] * 6 + [f32, vp]
    lib.fa_decode_paged_noalloc.restype = i32
    lib.fa_decode_paged_workspace_bytes.argtypes = [i32] * 5
    lib.fa_decode_paged_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [vp] * 10 + [i32, i32, i32, i32, f32, i32, vp, vp]
    lib.fa_bwd.restype = i32
    lib.fa_strerror.argtypes = [i32]
    lib.fa_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fa_strerror(status: int) -> str:
    return load_library().fa_strerror(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(nm, t, dtype, shape=None, device=None, contiguous=True):
    """Raise unless t is a tensor of ``dtype`` in device memory (on ``device``
    when given), contiguous unless told otherwise, of ``shape`` when given.
    Every pointer the library receives passes through here, so no host
    pointer, overlapping view or zero-stride expansion reaches a kernel."""
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != dtype:
        raise TypeError(f"{nm} must be a {dtype} tensor, got {getattr(t, 'dtype', type(t))}")
    if not t.is_cuda:
        raise ValueError(f"{nm} must be in device memory")
    if device is not None and t.device != device:
        raise ValueError(f"{nm} is on {t.device}, the other tensors on {device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{nm} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{nm} must be {list(shape)}, got {list(t.shape)}")


def _overlapping(t):
    """True if two index tuples of t address the same element: with its
    dimensions ordered by stride, each stride must be at least the span of
    the dimensions below it (dimensions of size 1 impose nothing)."""
    dims = sorted((st, n) for st, n in zip(t.stride(), t.shape) if n > 1)
    span = 1
    for st, n in dims:
        if st < span:
            return True
        span = st * (n - 1) + span
    return False


def _check_kv_lens(kv_lens, B, device):
    import torch
    if kv_lens is not None:
        _check("kv_lens", kv_lens, torch.int32, (B,), device)


def _call(name, q, k, v, o, lse, scale, mask_kind, kv_lens, stream, dtype):
    import torch
    lib = load_library()
    _check("q", q, dtype)
    if q.dim() != 4:
        raise ValueError(f"q must be [B, H, N, d], got {list(q.shape)}")
    for nm, t in (("k", k), ("v", v), ("o", o)):
        _check(nm, t, dtype, q.shape, q.device)
    B, H, N, d = q.shape
    _check("lse", lse, torch.float32, (B, H, N), q.device)
    _check_kv_lens(kv_lens, B, q.device)
    st = getattr(lib, name)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                            float(scale), int(mask_kind), _ptr(kv_lens),
                            ctypes.c_void_p(_stream_handle(stream, q.device)))
    if st != FA_OK:
        raise FaError(st, fa_strerror(st))


def fa_fwd(q, k, v, o, lse, scale, mask_kind=FA_MASK_NONE, kv_lens=None, stream=None):
    """bf16 forward: writes o (bf16) and lse (float32) on ``stream``."""
    import torch
    _call("fa_fwd", q, k, v, o, lse, scale, mask_kind, kv_lens, stream, torch.bfloat16)


def fa_fwd_f32(q, k, v, o, lse, scale, mask_kind=FA_MASK_NONE, kv_lens=None, stream=None):
    """float32 forward: writes o (float32) and lse (float32) on ``stream``."""
    import torch
    _call("fa_fwd_f32", q, k, v, o, lse, scale, mask_kind, kv_lens, stream, torch.float32)


def _stream_handle(stream, device):
    import torch
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def fa_fwd_general(q, k, v, o, lse, scale, mask_kind=FA_MASK_NONE, window_left=-1,
                   kv_lens=None, stream=None):
    """bf16 forward with Nq != Nk, a sliding window and strided views: q, o
    [B, H, Nq, d] and k, v [B, H, Nk, d] tensors (any strides whose last
    dimension is contiguous); lse contiguous float32 [B, H, Nq]."""
    import torch
    lib = load_library()
    _check("q", q, torch.bfloat16, contiguous=False)
    _check("k", k, torch.bfloat16, device=q.device, contiguous=False)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, Nq, d] and [B, H, Nk, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    strides = []
    for nm, t, rows in (("q", q, Nq), ("k", k, Nk), ("v", v, Nk), ("o", o, Nq)):
        _check(nm, t, torch.bfloat16, (B, H, rows, d), q.device, contiguous=False)
        if t.stride(3) != 1:
            raise ValueError(f"{nm} must have a contiguous last dimension")
        if nm == "o" and _overlapping(t):
            raise ValueError("o must not be an overlapping view (every element written once)")
        strides.append((ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2)))
    _check("lse", lse, torch.float32, (B, H, Nq), q.device)
    _check_kv_lens(kv_lens, B, q.device)
    st = lib.fa_fwd_general(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                            *[ctypes.cast(a, ctypes.c_void_p) for a in strides], float(scale),
                            int(mask_kind), int(window_left), _ptr(kv_lens),
                            ctypes.c_void_p(_stream_handle(stream, q.device)))
    if st != FA_OK:
        raise FaError(st, fa_strerror(st))


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, scale,
                  mask_kind=FA_MASK_NONE, window_left=-1, stream=None):
    """bf16 forward over packed sequences: q, o [total_q, H, d] and k, v
    [total_k, H, d] contiguous; lse float32 [H, total_q]; cu_seqlens_q/k
    int32 device tensors [B + 1] of sequence boundaries."""
    import torch
    lib = load_library()
    _check("q", q, torch.bfloat16)
    _check("k", k, torch.bfloat16, device=q.device)
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q and k must be [total_q, H, d] and [total_k, H, d]")
    total_q, H, d = q.shape
    total_k = k.shape[0]
    for nm, t, rows in (("q", q, total_q), ("k", k, total_k), ("v", v, total_k),
                        ("o", o, total_q)):
        _check(nm, t, torch.bfloat16, (rows, H, d), q.device)
    _check("lse", lse, torch.float32, (H, total_q), q.device)
    for nm, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        _check(nm, t, torch.int32, device=q.device)
        if t.dim() != 1:
            raise ValueError(f"{nm} must be [B + 1]")
    B = cu_seqlens_q.numel() - 1
    if B < 1 or cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 >= 2 entries")
    st = lib.fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens_q),
                           _ptr(cu_seqlens_k), B, H, d, total_q, total_k, int(max_seqlen_q),
                           float(scale), int(mask_kind), int(window_left),
                           ctypes.c_void_p(_stream_handle(stream, q.device)))
    if st != FA_OK:
        raise FaError(st, fa_strerror(st))


FP8_TILE = 128    # rows per scale tile of fa_fwd_fp8_tiled (FA_FP8_TILE)


def _fp8_call(name, q, k, v, q_descale, k_descale, v_descale, o, lse, scale, mask_kind,
              kv_lens, stream, qk_scales):
    import torch
    lib = load_library()
    _check("q", q, torch.uint8)    # E4M3 codes
    if q.dim() != 4:
        raise ValueError(f"q must be [B, H, N, d], got {list(q.shape)}")
    for nm, t in (("k", k), ("v", v)):
        _check(nm, t, torch.uint8, q.shape, q.device)
    B, H, N, d = q.shape
    for nm, t in (("q_descale", q_descale), ("k_descale", k_descale), ("v_descale", v_descale)):
        _check(nm, t, torch.float32, device=q.device)
        want = qk_scales(B, H, N) if nm != "v_descale" else B * H
        if t.numel() != want:
            raise ValueError(f"{nm} must hold {want} scales")
    _check("o", o, torch.bfloat16, (B, H, N, d), q.device)
    _check("lse", lse, torch.float32, (B, H, N), q.device)
    _check_kv_lens(kv_lens, B, q.device)
    st = getattr(lib, name)(_ptr(q), _ptr(k), _ptr(v), _ptr(q_descale), _ptr(k_descale),
                            _ptr(v_descale), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                            int(mask_kind), _ptr(kv_lens),
                            ctypes.c_void_p(_stream_handle(stream, q.device)))
    if st != FA_OK:
        raise FaError(st, fa_strerror(st))


def fa_fwd_fp8(q, k, v, q_descale, k_descale, v_descale, o, lse, scale, mask_kind=FA_MASK_NONE,
               kv_lens=None, stream=None):
    """E4M3 forward: q, k, v uint8 codes [B, H, N, d]; descales float32 [B, H];
    writes o (bf16) and lse (float32)."""
    _fp8_call("fa_fwd_fp8", q, k, v, q_descale, k_descale, v_descale, o, lse, scale, mask_kind,
              kv_lens, stream, lambda B, H, N: B * H)


def fa_fwd_fp8_tiled(q, k, v, q_descale, k_descale, v_descale, o, lse, scale,
                     mask_kind=FA_MASK_NONE, kv_lens=None, stream=None):
    """E4M3 forward with per-tile Q and K scales: q_descale, k_descale float32
    [B, H, ceil(N / 128)] (one per 128 rows), v_descale float32 [B, H]."""
    _fp8_call("fa_fwd_fp8_tiled", q, k, v, q_descale, k_descale, v_descale, o, lse, scale,
              mask_kind, kv_lens, stream, lambda B, H, N: B * H * (-(-N // FP8_TILE)))


def fa_decode_paged_workspace_bytes(B, H, d, block_size, max_blocks):
    return int(load_library().fa_decode_paged_workspace_bytes(B, H, d, block_size, max_blocks))


def fa_decode_paged(q, k_pool, v_pool, block_tables, seq_lens, o, lse, workspace, scale,
                    stream=None):
    """Decode over a paged KV cache: q bf16 [B, H, d]; pools bf16
    [num_blocks, H, block_size, d]; block_tables int32 [B, max_blocks];
    seq_lens int32 [B]; writes o (bf16 [B, H, d]) and lse (float32 [B, H])."""
    import torch
    lib = load_library()
    B, H, d, nblk, bs = _check_decode(q, k_pool, v_pool, block_tables, seq_lens, o, lse)
    need = fa_decode_paged_workspace_bytes(B, H, d, bs, block_tables.shape[1])
    _check("workspace", workspace, torch.float32, device=q.device)
    if workspace.numel() * 4 < need:
        raise ValueError(f"workspace must hold >= {need} bytes")
    st = lib.fa_decode_paged(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                             _ptr(seq_lens), _ptr(o), _ptr(lse), _ptr(workspace), B, H, d, bs,
                             block_tables.shape[1], nblk, float(scale),
                             ctypes.c_void_p(_stream_handle(stream, q.device)))
    if st != FA_OK:
        raise FaError(st, fa_strerror(st))

def _check_decode(q, k_pool, v_pool, block_tables, seq_lens, o, lse):
    import torch
    _check("q", q, torch.bfloat16)
    _check("k_pool", k_pool, torch.bfloat16, device=q.device)
    if q.dim() != 3 or k_pool.dim() != 4:
        raise ValueError("q must be [B, H, d] and the pools [num_blocks, H, block_size, d]")
    B, H, d = q.shape
    nblk, Hp, bs, dp = k_pool.shape
    if Hp != H or dp != d:
        raise ValueError("pools must be [num_blocks, H, block_size, d] with q's H and d")
    _check("v_pool", v_pool, torch.bfloat16, k_pool.shape, q.device)
    _check("o", o, torch.bfloat16, (B, H, d), q.device)
    _check("block_tables", block_tables, torch.int32, device=q.device)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks]")
    _check("seq_lens", seq_lens, torch.int32, (B,), q.device)
    _check("lse", lse, torch.float32, (B, H), q.device)
    return B, H, d, nblk, bs


def fa_decode_paged_noalloc(q, k_pool, v_pool, block_tables, seq_lens, o, lse, scale,
                            stream=None):
    """fa_decode_paged without a workspace: the partial results live in the
    library's fixed per-GPU buffer (DECODE_NOALLOC_SCRATCH_BYTES); for
    callers that cannot allocate.  Calls that may overlap on one GPU race."""
    lib = load_library()
    B, H, d, nblk, bs = _check_decode(q, k_pool, v_pool, block_tables, seq_lens, o, lse)
    st = lib.fa_decode_paged_noalloc(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                     _ptr(seq_lens), _ptr(o), _ptr(lse), B, H, d, bs,
                                     block_tables.shape[1], nblk, float(scale),
                                     ctypes.c_void_p(_stream_handle(stream, q.device)))
    if st != FA_OK:
        raise FaError(st, fa_strerror(st))

def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, dp_rowsum, scale, mask_kind=FA_MASK_NONE,
           kv_lens=None, stream=None):
    """bf16 backward: writes dq, dk, dv (bf16) and dp_rowsum (float32 [B, H, N])."""
    import torch
    lib = load_library()
    _check("q", q, torch.bfloat16)
    if q.dim() != 4:
        raise ValueError(f"q must be [B, H, N, d], got {list(q.shape)}")
    for nm, t in (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk),
                  ("dv", dv)):
        _check(nm, t, torch.bfloat16, q.shape, q.device)
    B, H, N, d = q.shape
    for nm, t in (("lse", lse), ("dp_rowsum", dp_rowsum)):
        _check(nm, t, torch.float32, (B, H, N), q.device)
    _check_kv_lens(kv_lens, B, q.device)
    st = lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                    _ptr(dk), _ptr(dv), _ptr(dp_rowsum), B, H, N, d, float(scale),
                    int(mask_kind), _ptr(kv_lens),
                    ctypes.c_void_p(_stream_handle(stream, q.device)))
    if st != FA_OK:
        raise FaError(st, fa_strerror(st))


def attention_grad(q, k, v, o, lse, dout, scale=None, mask_kind=FA_MASK_NONE, kv_lens=None,
                   stream=None):
    """Allocate the gradients and run the backward pass; returns ``(dq, dk, dv)``."""
    import torch
    B, H, N, d = q.shape
    if scale is None:
        scale = d ** -0.5
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dps = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, dps, scale, mask_kind, kv_lens, stream)
    return dq, dk, dv


def attention(q, k, v, scale=None, mask_kind=FA_MASK_NONE, kv_lens=None, stream=None):
    """Allocate O and LSE and run the forward pass; returns ``(o, lse)``."""
    import torch
    B, H, N, d = q.shape
    if scale is None:
        scale = d ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fn = fa_fwd if q.dtype == torch.bfloat16 else fa_fwd_f32
    fn(q, k, v, o, lse, scale, mask_kind, kv_lens, stream)
    return o, lse
