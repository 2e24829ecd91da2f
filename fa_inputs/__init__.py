"""Seeded synthetic inputs for the attention forward and backward passes.

This module only draws and encodes numbers: it holds none of the attention
arithmetic.  Both the CPU oracle's tests and the GPU path's tests and bench
take their inputs from here, so that both sides consume the same bytes.

Recipe (identical for every workload):

* ``numpy.random.SeedSequence(seed).spawn(4)`` gives four independent PCG64
  streams, used for Q, K, V and the per-batch key lengths, in that order.
* Q, K, V are ``standard_normal`` draws in float32, shaped ``[B, H, N, d]``
  (contiguous, row-major).  Q is multiplied by ``q_mult`` (a power of two, so
  the product is exact in binary floating point).
* bf16 workloads convert the float32 draws to bfloat16 with
  round-to-nearest-even and keep them as uint16 bit patterns.
* Key-padding workloads draw one valid key length per batch entry,
  uniform over the inclusive integer range ``kv_len_range``.
* The backward pass's upstream gradient dO (same shape as O) comes from a
  fifth stream, ``SeedSequence(seed).spawn(5)[4]`` (the first four children
  are the ones above, so the forward inputs do not change): float32
  ``standard_normal``, then bf16 as above for bf16 workloads.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_KEY_PADDING = 2


@dataclass(frozen=True)
class Workload:
    """One attention forward workload: shapes, dtype, mask and input recipe."""

    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32" or "bf16"
    mask_kind: int
    seed: int
    q_mult: float = 1.0
    kv_len_range: Optional[Tuple[int, int]] = None
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        # 1/sqrt(d), rounded to the float32 value the kernel receives.
        return float(np.float32(1.0 / np.sqrt(self.d)))

    def flops(self) -> float:
        """Forward FLOPs by the metric's formula: 4*B*H*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if (self.mask_kind & MASK_CAUSAL) else f

    def bwd_flops(self) -> float:
        """Backward FLOPs by the same convention: the five products of the
        gradient (S, dP, dV, dQ, dK; 2*N^2*d each), i.e. 2.5x the forward."""
        return 2.5 * self.flops()


# The five workloads the parity tests and the bench use.  Seeds are fixed per
# workload; the two runs of the B=4,H=16 workload share inputs.
WORKLOADS = {
    "f32_b1h1_n256_d64": Workload(
        "f32_b1h1_n256_d64", 1, 1, 256, 64, "f32", MASK_NONE, seed=1,
        note="single head, fp32, unmasked"),
    "bf16_b4h16_n1024_d64": Workload(
        "bf16_b4h16_n1024_d64", 4, 16, 1024, 64, "bf16", MASK_NONE, seed=2,
        note="unmasked"),
    "bf16_b4h16_n1024_d64_causal": Workload(
        "bf16_b4h16_n1024_d64_causal", 4, 16, 1024, 64, "bf16", MASK_CAUSAL, seed=2,
        note="causal, same inputs as the unmasked run"),
    "bf16_b2h32_n4096_d128_causal": Workload(
        "bf16_b2h32_n4096_d128_causal", 2, 32, 4096, 128, "bf16", MASK_CAUSAL, seed=3,
        q_mult=2.0, note="causal, Q ~ 2*N(0,1) so the running max moves often"),
    "bf16_b8h16_n2048_d64_keypad": Workload(
        "bf16_b8h16_n2048_d64_keypad", 8, 16, 2048, 64, "bf16", MASK_KEY_PADDING, seed=4,
        kv_len_range=(1024, 2048), note="key padding, kv_len ~ U{1024..2048}"),
    "bf16_b1h8_n65536_d128_causal": Workload(
        "bf16_b1h8_n65536_d128_causal", 1, 8, 65536, 128, "bf16", MASK_CAUSAL, seed=5,
        note="long context, causal"),
}

# The workload the throughput figure is quoted on.
BENCH_WORKLOAD = "bf16_b2h32_n4096_d128_causal"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    NaN inputs map to a quiet NaN.  This is an input encoding step, not part
    of the attention arithmetic.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32)


def _streams(seed: int, n: int = 4):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(n)]


def make_raw(B: int, H: int, N: int, d: int, dtype: str, seed: int,
             q_mult: float = 1.0, kv_len_range: Optional[Tuple[int, int]] = None):
    """Draw Q, K, V (and kv_lens) for an arbitrary shape.

    Returns a dict with ``q``, ``k``, ``v`` (float32 arrays for ``"f32"``,
    uint16 bf16 bit patterns for ``"bf16"``) and ``kv_lens`` (int32 ``[B]`` or
    None).
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    gq, gk, gv, gl = _streams(seed)
    shape = (B, H, N, d)
    q = gq.standard_normal(shape, dtype=np.float32)
    if q_mult != 1.0:
        q *= np.float32(q_mult)
    k = gk.standard_normal(shape, dtype=np.float32)
    v = gv.standard_normal(shape, dtype=np.float32)
    kv_lens = None
    if kv_len_range is not None:
        lo, hi = kv_len_range
        kv_lens = gl.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    if dtype == "bf16":
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    return {"q": q, "k": k, "v": v, "kv_lens": kv_lens}


def make_grad_out(B: int, H: int, N: int, d: int, dtype: str, seed: int):
    """Draw the upstream gradient dO ``[B, H, N, d]`` for the backward pass."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    g = _streams(seed, 5)[4]
    do = g.standard_normal((B, H, N, d), dtype=np.float32)
    return f32_to_bf16_bits(do) if dtype == "bf16" else do


def make_inputs(wl: Workload):
    """Draw the inputs of a named workload (see ``WORKLOADS``)."""
    return make_raw(wl.B, wl.H, wl.N, wl.d, wl.dtype, wl.seed,
                    q_mult=wl.q_mult, kv_len_range=wl.kv_len_range)


def make_bwd_inputs(wl: Workload):
    """The forward inputs of a workload plus its upstream gradient ``do``."""
    x = make_inputs(wl)
    x["do"] = make_grad_out(wl.B, wl.H, wl.N, wl.d, wl.dtype, wl.seed)
    return x


def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact float64 view of generated data (bf16 bit patterns or float32)."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)
