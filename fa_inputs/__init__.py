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
* fp8 workloads quantize the same float32 draws to OCP FP8 E4M3 (the
  "e4m3fn" encoding: 4 exponent bits with bias 7, 3 mantissa bits, largest
  finite value 448, no infinities) with one float32 scale per (batch, head)
  and tensor: descale = max|x| / 448 over that head's [N, d] values, code =
  nearest E4M3 value of x / descale (ties to the even code).  The
  dequantized value is code_value * descale.
* Paged decode (one query token per request against a paged KV cache):
  ``SeedSequence(seed).spawn(5)`` streams for q, the K pool, the V pool,
  the request lengths and the block placement.  Lengths are uniform over the
  inclusive ``len_range``; request b needs ceil(n_b / block_size) blocks;
  the pool holds exactly those blocks plus ``spare`` unused ones, placed by
  a random permutation (so a request's blocks are scattered through the
  pool); table entries past a request's last block hold -1.  q and both
  pools are float32 N(0,1) rounded to bf16, pools shaped
  [num_blocks, H, block_size, d].
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
    dtype: str  # "f32", "bf16" or "fp8"
    mask_kind: int
    seed: int
    q_mult: float = 1.0
    kv_len_range: Optional[Tuple[int, int]] = None
    note: str = field(default="", compare=False)
    window_left: int = -1      # sliding window (general forward only)
    layout: str = "bhnd"       # "bnhd": tensors stored [B, N, H, d] (general forward only);
    #                            "varlen": B packed sequences, lengths U[len_range] (N = max)
    len_range: Optional[Tuple[int, int]] = None
    tile_gain: Optional[float] = None   # fp8 only: quantize Q, K per 128-row tile (make_raw_fp8_tiled)

    @property
    def scale(self) -> float:
        # 1/sqrt(d), rounded to the float32 value the kernel receives.
        return float(np.float32(1.0 / np.sqrt(self.d)))

    def flops(self) -> float:
        """Forward FLOPs by the metric's formula: 4*B*H*N^2*d, halved when causal.
        With a sliding window: 4*d per visible (query, key) pair.  Packed
        sequences: the same count summed over the sequences (n^2, or
        n(n+1)/2 causal)."""
        if self.layout == "varlen":
            n = packed_lengths(self).astype(np.float64)
            pairs = n * (n + 1) / 2.0 if self.mask_kind & MASK_CAUSAL else n * n
            return 4.0 * self.H * self.d * float(pairs.sum())
        if self.window_left >= 0:
            W, N = self.window_left, self.N
            if self.mask_kind & MASK_CAUSAL:
                pairs = (W + 1) * N - W * (W + 1) / 2.0 if W < N else N * (N + 1) / 2.0
            else:
                pairs = sum(N - max(0, r - W) for r in range(N))
            return 4.0 * self.B * self.H * pairs * self.d
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

# The fp8 counterpart of the bench workload: the same draws, quantized per head.
FP8_WORKLOADS = {
    "fp8_b2h32_n4096_d128_causal": Workload(
        "fp8_b2h32_n4096_d128_causal", 2, 32, 4096, 128, "fp8", MASK_CAUSAL, seed=3,
        q_mult=2.0, note="fp8 E4M3 Q, K, V with per-head scales; causal"),
    "fp8_tiled_b2h32_n4096_d128_causal": Workload(
        "fp8_tiled_b2h32_n4096_d128_causal", 2, 32, 4096, 128, "fp8", MASK_CAUSAL, seed=3,
        q_mult=2.0, tile_gain=3.0,
        note="fp8 E4M3 Q, K with one scale per 128 rows (tile ranges spread over 2^[-3, 3]), "
             "V per head; causal"),
}

@dataclass(frozen=True)
class DecodeWorkload:
    """One paged-KV decode workload (one query token per request)."""

    name: str
    B: int
    H: int
    d: int
    block_size: int
    len_range: Tuple[int, int]
    seed: int
    spare: int = 16

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.d)))


DECODE_WORKLOADS = {
    "decode_b32h32_d128_bs64_len1k8k": DecodeWorkload(
        "decode_b32h32_d128_bs64_len1k8k", 32, 32, 128, 64, (1024, 8192), seed=6),
}


# Workloads of the general forward (strided layouts, sliding windows).
GENERAL_WORKLOADS = {
    "bf16_b1h8_n65536_d128_causal_w4096": Workload(
        "bf16_b1h8_n65536_d128_causal_w4096", 1, 8, 65536, 128, "bf16", MASK_CAUSAL, seed=5,
        window_left=4096, note="long context, causal, sliding window of 4096 keys"),
    "bf16_b2h32_n4096_d128_causal_bnhd": Workload(
        "bf16_b2h32_n4096_d128_causal_bnhd", 2, 32, 4096, 128, "bf16", MASK_CAUSAL, seed=3,
        q_mult=2.0, layout="bnhd", note="the bench workload stored [B, N, H, d]"),
    "bf16_varlen_b16h32_n512_4096_d128_causal": Workload(
        "bf16_varlen_b16h32_n512_4096_d128_causal", 16, 32, 4096, 128, "bf16", MASK_CAUSAL,
        seed=8, q_mult=2.0, layout="varlen", len_range=(512, 4096),
        note="16 packed causal sequences, lengths uniform in [512, 4096]"),
}


def packed_lengths(wl: "Workload") -> np.ndarray:
    """The B sequence lengths of a packed workload (seeded, uniform in
    ``len_range``; the longest is set to N so max_seqlen is exactly N)."""
    lo, hi = wl.len_range
    n = _streams(wl.seed)[3].integers(lo, hi, size=wl.B, endpoint=True).astype(np.int64)
    n[int(np.argmax(n))] = wl.N
    return n

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


def _fp8_decode_code(c: int) -> float:
    """Value of an E4M3 (e4m3fn) code with the sign bit clear (0..126)."""
    e, m = c >> 3, c & 7
    if e == 0:
        return m * 2.0 ** -9               # subnormal: 2^-6 * m/8
    return (1.0 + m / 8.0) * 2.0 ** (e - 7)


# Non-negative E4M3 values by code 0..126 (0x7F is NaN); increasing in the code.
_FP8_POS = np.array([_fp8_decode_code(c) for c in range(0x7F)], dtype=np.float64)
FP8_MAX = 448.0


def f32_to_fp8_e4m3(x: np.ndarray) -> np.ndarray:
    """float -> E4M3 codes (uint8): the nearest representable value, ties to
    the even code (the one whose mantissa ends in 0).  |x| above 448 is
    clamped to 448 (the recipe scales values into range first).  An input
    encoding step, not attention arithmetic."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), FP8_MAX)
    hi = np.clip(np.searchsorted(_FP8_POS, a, side="left"), 0, len(_FP8_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _FP8_POS[lo]
    dhi = _FP8_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(x)             # a negative value that rounds to 0 keeps its sign
    return (code | (neg.astype(np.uint8) << 7)).astype(np.uint8)


def fp8_e4m3_to_f64(u: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) -> exact float64 values (0x7F/0xFF decode as NaN)."""
    u = np.asarray(u, dtype=np.uint8)
    mag = np.concatenate([_FP8_POS, [np.nan]])[u & 0x7F]
    return np.where(u & 0x80, -mag, mag)


def quantize_fp8_per_head(x: np.ndarray):
    """Per-(batch, head) E4M3 quantization of float32 [B, H, N, d]: returns
    (codes uint8 [B, H, N, d], descale float32 [B, H])."""
    amax = np.abs(x).max(axis=(2, 3)).astype(np.float32)
    descale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    codes = f32_to_fp8_e4m3(x.astype(np.float64) / descale[:, :, None, None].astype(np.float64))
    return codes, descale


def dequant_fp8_f64(codes: np.ndarray, descale: np.ndarray) -> np.ndarray:
    """Exact float64 values code_value * descale of per-head quantized data."""
    return fp8_e4m3_to_f64(codes) * np.asarray(descale, dtype=np.float64)[:, :, None, None]


FP8_TILE = 128   # rows per scale tile of the tiled fp8 entry point


def _tile_rows(descale: np.ndarray, N: int, tile: int) -> np.ndarray:
    """Per-row scale [B, H, N] from per-tile scales [B, H, ceil(N / tile)]."""
    return np.repeat(np.asarray(descale), tile, axis=2)[:, :, :N]


def quantize_fp8_per_tile(x: np.ndarray, tile: int = FP8_TILE):
    """E4M3 quantization of float32 [B, H, N, d] with one scale per ``tile``
    consecutive rows of each (batch, head): returns (codes uint8 [B, H, N, d],
    descale float32 [B, H, ceil(N / tile)])."""
    B, H, N, d = x.shape
    T = -(-N // tile)
    padded = np.zeros((B, H, T * tile, d), dtype=np.float32)
    padded[:, :, :N] = x
    amax = np.abs(padded.reshape(B, H, T, tile * d)).max(axis=3).astype(np.float32)
    descale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    rows = _tile_rows(descale, N, tile).astype(np.float64)
    return f32_to_fp8_e4m3(x.astype(np.float64) / rows[..., None]), descale


def dequant_fp8_tiled_f64(codes: np.ndarray, descale: np.ndarray,
                          tile: int = FP8_TILE) -> np.ndarray:
    """Exact float64 values code_value * descale of per-tile quantized data."""
    rows = _tile_rows(np.asarray(descale, dtype=np.float64), codes.shape[2], tile)
    return fp8_e4m3_to_f64(codes) * rows[..., None]


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
    if dtype not in ("f32", "bf16", "fp8"):
        raise ValueError(f"dtype must be 'f32', 'bf16' or 'fp8', got {dtype!r}")
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
    if dtype == "fp8":
        (q, qs), (k, ks), (v, vs) = (quantize_fp8_per_head(t) for t in (q, k, v))
        return {"q": q, "k": k, "v": v, "kv_lens": kv_lens,
                "q_descale": qs, "k_descale": ks, "v_descale": vs}
    return {"q": q, "k": k, "v": v, "kv_lens": kv_lens}


def make_raw_fp8_tiled(B: int, H: int, N: int, d: int, seed: int, q_mult: float = 1.0,
                      kv_len_range: Optional[Tuple[int, int]] = None, tile_gain: float = 0.0):
    """The draws of ``make_raw`` with Q and K quantized per FP8_TILE-row tile
    (descales [B, H, ceil(N / FP8_TILE)]) and V per head.  With ``tile_gain``
    > 0 every row tile of Q and of K is first multiplied by 2^u, u uniform in
    [-tile_gain, tile_gain] (its own stream), so the tiles span different
    ranges -- the case block quantization is for."""
    gq, gk, gv, gl, gg = _streams(seed, 5)
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
    T = -(-N // FP8_TILE)
    if tile_gain > 0:
        for t in (q, k):
            u = gg.uniform(-tile_gain, tile_gain, size=(B, H, T))
            t *= _tile_rows(np.exp2(u), N, FP8_TILE)[..., None].astype(np.float32)
    (qc, qs), (kc, ks) = quantize_fp8_per_tile(q), quantize_fp8_per_tile(k)
    vc, vs = quantize_fp8_per_head(v)
    return {"q": qc, "k": kc, "v": vc, "kv_lens": kv_lens, "q_descale": qs, "k_descale": ks,
            "v_descale": vs, "fp8_tiled": True, "q_f32": q, "k_f32": k, "v_f32": v}


def make_packed(lens_q, lens_k, H: int, d: int, seed: int, q_mult: float = 1.0):
    """Packed variable-length bf16 inputs: q ``[total_q, H, d]``, k, v
    ``[total_k, H, d]`` (bf16 bit patterns, N(0, 1) draws rounded to bf16,
    q scaled by ``q_mult`` first) and the boundaries cu_q, cu_k (int32
    ``[B + 1]``, cumulative lengths starting at 0)."""
    lens_q = np.asarray(lens_q, dtype=np.int64)
    lens_k = np.asarray(lens_k, dtype=np.int64)
    if lens_q.shape != lens_k.shape or (lens_q < 0).any() or (lens_k < 0).any():
        raise ValueError("lens_q and lens_k must be equally long lists of lengths >= 0")
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    gq, gk, gv, _ = _streams(seed)
    q = gq.standard_normal((int(cu_q[-1]), H, d), dtype=np.float32)
    if q_mult != 1.0:
        q *= np.float32(q_mult)
    k = gk.standard_normal((int(cu_k[-1]), H, d), dtype=np.float32)
    v = gv.standard_normal((int(cu_k[-1]), H, d), dtype=np.float32)
    return {"q": f32_to_bf16_bits(q), "k": f32_to_bf16_bits(k), "v": f32_to_bf16_bits(v),
            "cu_q": cu_q, "cu_k": cu_k}


def make_grad_out(B: int, H: int, N: int, d: int, dtype: str, seed: int):
    """Draw the upstream gradient dO ``[B, H, N, d]`` for the backward pass."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    g = _streams(seed, 5)[4]
    do = g.standard_normal((B, H, N, d), dtype=np.float32)
    return f32_to_bf16_bits(do) if dtype == "bf16" else do


def make_paged_decode(B: int, H: int, d: int, block_size: int, len_range, seed: int,
                      spare: int = 16, lens=None):
    """Draw a paged-KV decode batch (see the recipe above).  Returns a dict:
    ``q`` [B, H, d], ``k_pool``/``v_pool`` [num_blocks, H, block_size, d]
    (bf16 bits), ``block_tables`` int32 [B, max_blocks], ``seq_lens`` int32 [B].
    ``lens`` (optional) replaces the drawn lengths."""
    gq, gk, gv, gl, gp = _streams(seed, 5)
    lo, hi = len_range
    drawn = gl.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    lens = drawn if lens is None else np.asarray(lens, dtype=np.int32)
    nblk = (lens.astype(np.int64) + block_size - 1) // block_size
    max_blocks = max(1, int(nblk.max()))
    num_blocks = int(nblk.sum()) + spare
    perm = gp.permutation(num_blocks).astype(np.int32)
    tables = np.full((B, max_blocks), -1, dtype=np.int32)
    at = 0
    for b in range(B):
        tables[b, :nblk[b]] = perm[at:at + nblk[b]]
        at += int(nblk[b])
    shape = (num_blocks, H, block_size, d)

    def pool(g):
        out = np.empty(shape, dtype=np.uint16)
        for i in range(0, num_blocks, 256):          # in chunks: bounded float32 staging
            j = min(num_blocks, i + 256)
            out[i:j] = f32_to_bf16_bits(g.standard_normal((j - i,) + shape[1:], dtype=np.float32))
        return out

    q = f32_to_bf16_bits(gq.standard_normal((B, H, d), dtype=np.float32))
    return {"q": q, "k_pool": pool(gk), "v_pool": pool(gv), "block_tables": tables,
            "seq_lens": lens}


def make_inputs(wl: Workload):
    """Draw the inputs of a named workload (see ``WORKLOADS``)."""
    if wl.layout == "varlen":
        n = packed_lengths(wl)
        return make_packed(n, n, wl.H, wl.d, wl.seed, q_mult=wl.q_mult)
    if wl.tile_gain is not None:
        return make_raw_fp8_tiled(wl.B, wl.H, wl.N, wl.d, wl.seed, q_mult=wl.q_mult,
                                  kv_len_range=wl.kv_len_range, tile_gain=wl.tile_gain)
    return make_raw(wl.B, wl.H, wl.N, wl.d, wl.dtype, wl.seed,
                    q_mult=wl.q_mult, kv_len_range=wl.kv_len_range)


def make_bwd_inputs(wl: Workload):
    """The forward inputs of a workload plus its upstream gradient ``do``."""
    x = make_inputs(wl)
    x["do"] = make_grad_out(wl.B, wl.H, wl.N, wl.d, wl.dtype, wl.seed)
    return x


def inputs_f64(x: dict):
    """Exact float64 Q, K, V of a generated input dict (any dtype)."""
    if x["q"].dtype == np.uint8 and x.get("fp8_tiled"):
        return (dequant_fp8_tiled_f64(x["q"], x["q_descale"]),
                dequant_fp8_tiled_f64(x["k"], x["k_descale"]),
                dequant_fp8_f64(x["v"], x["v_descale"]))
    if x["q"].dtype == np.uint8:
        return tuple(dequant_fp8_f64(x[n], x[n + "_descale"]) for n in "qkv")
    return tuple(to_f64(x[n]) for n in "qkv")


def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact float64 view of generated data (bf16 bit patterns or float32)."""
    if x.dtype == np.uint8:
        raise ValueError("fp8 codes need their scales: use inputs_f64 / dequant_fp8_f64")
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)
