"""Exact attention forward on MI355X (gfx950): Python binding of libfa92.so.

The binding only marshals arguments: every step of the forward pass runs in
the HIP kernels of ``csrc/fa_fwd.hip``.  PyTorch supplies device memory and
the stream.  There is no CPU or PyTorch fallback: if the library is missing
or the GPU is absent, the calls raise.

Names follow the C ABI of ``include/fa_api.h``:

* ``fa_fwd(q, k, v, o, lse, scale, mask_kind=0, kv_lens=None, stream=None)``
  -- bf16 tensors ``[B, H, N, d]``
* ``fa_fwd_f32(...)`` -- the same with float32 tensors
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

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa92.so")
EXPORTS = ("fa_fwd", "fa_fwd_f32", "fa_strerror")

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
    lib.fa_strerror.argtypes = [i32]
    lib.fa_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fa_strerror(status: int) -> str:
    return load_library().fa_strerror(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _call(name, q, k, v, o, lse, scale, mask_kind, kv_lens, stream, dtype):
    import torch
    lib = load_library()
    for nm, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t.dtype != dtype:
            raise TypeError(f"{nm} must be {dtype}, got {t.dtype}")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous device tensor")
        if t.dim() != 4 or t.shape != q.shape:
            raise ValueError(f"{nm} must have the shape of q, [B, H, N, d]")
    B, H, N, d = q.shape
    if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous() \
            or tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be a contiguous float32 device tensor [B, H, N]")
    if kv_lens is not None:
        if kv_lens.dtype != torch.int32 or not kv_lens.is_cuda or kv_lens.numel() != B:
            raise ValueError("kv_lens must be an int32 device tensor [B]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    st = getattr(lib, name)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                            float(scale), int(mask_kind), _ptr(kv_lens),
                            ctypes.c_void_p(stream))
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
