"""CPU oracle for the gradients of exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the package's smoke check and the
bench's CPU-baseline leg use it.  It shares no code with the HIP kernels.

Sources (web pages; cited by title and section):

* [G]  "FlashAttention算法详解：从IO瓶颈到Triton实现" (gentlecold.top),
       section Backward为什么更复杂
* [Y]  FlashAttention paper walkthrough, flash_attention.zh (youngju.dev),
       §7 (recomputation in the backward pass)

What is computed.  With S = scale * Q K^T + M (M = 0 on the visible keys
J_r of row r, -inf elsewhere; the same masks as the forward oracle) and
P = softmax(S) row by row, an upstream gradient dO of O = P V gives
([G] Backward为什么更复杂, the five gradient equations):

    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - rowsum(dP * P))        (* is the elementwise product)
    dQ = scale * dS K
    dK = scale * dS^T Q

The pages write dQ = dS K and dK = dS^T Q for scores S = Q K^T; here the
scores carry the softmax scale, so the chain rule multiplies both by
``scale`` (dV has no scale).  The row sum rowsum(dP * P) is also returned
as ``dp_rowsum`` (one fp32 value per query row on the kernel side).

``attention_bwd_ref`` is that definition, fp64 throughout: P is computed
afresh from Q and K with the max-subtracted softmax, never from saved
statistics, one block of query rows at a time (the row blocking only
bounds memory; every element's arithmetic is a plain sum of products).

``blocked_attention_bwd_ref`` follows the pages' recomputation scheme
([G] Backward为什么更复杂, the flowchart; [Y] §7.2): the forward keeps only
O and the per-row LSE; the backward visits (query block, key block) pairs,
rebuilds each block's probabilities as P_ij = exp(S_ij - LSE_i) and adds
into dV, dQ and dK.  It needs rowsum(dP * P) before the scan; the pages do
not say where it comes from.  Reading: it equals rowsum(dO * O), because
sum_c P_rc (dO_r . v_c) = dO_r . (sum_c P_rc v_c) = dO_r . O_r.  That
function exists to pin the recomputation (any partition and visiting order
gives the definition's result), not for parity.

Readings where the pages are silent:

* A query row with no visible key (kv_len = 0) has P_r = 0, so it adds
  nothing to dK, dV and has dQ_r = 0; its dp_rowsum is 0.
* Keys that no row sees (beyond kv_len, or past every row under the causal
  mask) get dK = dV = 0.
* ``scale`` is the float32 value a kernel receives, widened to float64.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from typing import Iterable, Optional

import numpy as np

from .attention_ref import MASK_CAUSAL, MASK_KEY_PADDING, partition

_MASK_BITS = MASK_CAUSAL | MASK_KEY_PADDING


def _as_scale(scale: float) -> float:
    return float(np.float32(scale))


def _visible(rows, cols, causal, n_vis):
    vis = cols[None, :] < n_vis
    if causal:
        vis = vis & (cols[None, :] <= rows[:, None])
    return np.broadcast_to(vis, (len(rows), len(cols)))


def _head_bwd(qh, kh, vh, doh, scale, causal, n_vis, rows, row_block, mags):
    """dQ, dK, dV and rowsum(dP * P) of one (b, h), by the definition, with
    the contributions of the query rows ``rows`` (sorted).  When ``mags`` is
    a dict, it also receives the magnitudes described in attention_bwd_ref."""
    N, d = qh.shape
    dq = np.full((N, d), np.nan)
    dk = np.zeros((N, d))
    dv = np.zeros((N, d))
    dps = np.full(N, np.nan)
    dq[rows] = 0.0
    dps[rows] = 0.0
    if mags is not None:
        mags.update(dq=np.full((N, d), np.nan), dk=np.zeros((N, d)), dv=np.zeros((N, d)),
                    dps=np.full(N, np.nan))
        mags["dq"][rows] = 0.0
        mags["dps"][rows] = 0.0
    for start in range(0, len(rows), row_block):
        rr = rows[start:start + row_block]
        kmax = min(n_vis, int(rr[-1]) + 1) if causal else n_vis
        if kmax <= 0:
            continue
        cols = np.arange(kmax)
        s = (qh[rr] @ kh[:kmax].T) * scale
        s = np.where(_visible(rr, cols, causal, n_vis), s, -np.inf)
        m = s.max(axis=1)
        ok = np.isfinite(m)                       # rows with >= 1 visible key
        p = np.zeros_like(s)
        e = np.exp(s[ok] - m[ok, None])
        p[ok] = e / e.sum(axis=1, keepdims=True)  # P = softmax(S), masked -> 0
        dv[:kmax] += p.T @ doh[rr]                # dV = P^T dO
        dp = doh[rr] @ vh[:kmax].T                # dP = dO V^T
        rs = (dp * p).sum(axis=1)                 # rowsum(dP * P)
        ds = p * (dp - rs[:, None])               # dS = P * (dP - rowsum)
        dq[rr] = (ds @ kh[:kmax]) * scale         # dQ = scale dS K
        dk[:kmax] += (ds.T @ qh[rr]) * scale      # dK = scale dS^T Q
        dps[rr] = rs
        if mags is not None:
            aq, ak, av, ado = (np.abs(t) for t in (qh[rr], kh[:kmax], vh[:kmax], doh[rr]))
            ads = np.abs(ds)
            a_d = (ado * (p @ av)).sum(axis=1)            # sum_t |dO| (P |V|)
            mags["dps"][rr] = a_d
            mags["dv"][:kmax] += p.T @ ado
            sa = abs(scale)                               # |scale * term| = |scale| |term|
            mags["dq"][rr] = sa * (ads @ ak + a_d[:, None] * (p @ ak))
            mags["dk"][:kmax] += sa * (ads.T @ aq + p.T @ (a_d[:, None] * aq))
    return dq, dk, dv, dps


def _check(q, k, v, do, mask_kind, kv_lens):
    B, H, N, d = q.shape
    for t in (k, v, do):
        if t.shape != (B, H, N, d):
            raise ValueError("q, k, v, do must share the shape [B, H, N, d]")
    if mask_kind & ~_MASK_BITS:
        raise ValueError(f"unknown mask bits in {mask_kind}")
    if (mask_kind & MASK_KEY_PADDING) and kv_lens is None:
        raise ValueError("key padding needs kv_lens")


def _n_vis(mask_kind, kv_lens, b, N):
    if mask_kind & MASK_KEY_PADDING:
        return max(0, min(int(kv_lens[b]), N))
    return N


def attention_bwd_ref(q, k, v, do, scale, mask_kind=0, kv_lens=None, heads=None,
                      rows=None, row_block: int = 512, workers: int = 1,
                      magnitudes: bool = False):
    """fp64 gradients of exact attention.

    q, k, v, do: float64 ``[B, H, N, d]``.  ``heads``: optional list of
    (b, h) pairs to compute (default all; the others stay NaN).  ``rows``:
    optional sorted query-row indices; only those rows' terms are summed, so
    dQ and dp_rowsum are exact on them (NaN elsewhere) and dK, dV are exact
    for every key that no other row sees (under the causal mask: every key
    at or after the first row of a contiguous tail ``rows``).  Returns
    ``dQ, dK, dV`` (``[B, H, N, d]``) and ``dp_rowsum`` (``[B, H, N]``).

    ``magnitudes=True`` appends a dict of the same four shapes holding, for
    each element, the sum of the absolute values of the terms a finite-
    precision evaluation adds up (the quantity rounding-error bounds of
    sums scale with; for tolerances only):

        dv:  P^T |dO|
        dps: sum_t |dO_rt| (P |V|)_rt          (bounds rowsum(dO * O) too)
        dq:  |scale| (|dS| |K| + dps_mag_r * P |K|)
        dk:  |scale| (|dS|^T |Q| + P^T (dps_mag * |Q|))

    The second terms carry an error of the row sum into dS = P (dP - D).
    """
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    _check(q, k, v, do, mask_kind, kv_lens)
    B, H, N, d = q.shape
    scale = _as_scale(scale)
    causal = bool(mask_kind & MASK_CAUSAL)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    units = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    dQ, dK, dV = (np.full((B, H, N, d), np.nan) for _ in range(3))
    DP = np.full((B, H, N), np.nan)
    M = ({"dq": np.full((B, H, N, d), np.nan), "dk": np.full((B, H, N, d), np.nan),
          "dv": np.full((B, H, N, d), np.nan), "dps": np.full((B, H, N), np.nan)}
         if magnitudes else None)

    def run(unit):
        b, h = unit
        n_vis = _n_vis(mask_kind, kv_lens, b, N)
        mags = {} if magnitudes else None
        dQ[b, h], dK[b, h], dV[b, h], DP[b, h] = _head_bwd(
            q[b, h], k[b, h], v[b, h], do[b, h], scale, causal, n_vis, rows, row_block, mags)
        if magnitudes:
            for name in M:
                M[name][b, h] = mags[name]

    if workers <= 1 or len(units) == 1:
        for u in units:
            run(u)
    else:
        # Parallel over independent heads only; BLAS held to one thread each.
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
            list(ex.map(run, units))
    if magnitudes:
        return dQ, dK, dV, DP, M
    return dQ, dK, dV, DP


def blocked_attention_bwd_ref(q, k, v, o, lse, do, scale, mask_kind=0, kv_len=None,
                              q_blocks: Optional[Iterable[np.ndarray]] = None,
                              k_blocks: Optional[Iterable[np.ndarray]] = None,
                              key_outer: bool = True):
    """One head's gradients by the block scan with recomputed probabilities.

    q, k, v, o, do: ``[N, d]`` float64; lse: ``[N]`` (natural log, -inf for
    rows with no visible key).  Blocks may be any partitions of 0..N-1 in
    any order; ``key_outer`` picks which index the outer loop runs over.
    Per pair (query block i, key block j):

        qk  = scale Q_i K_j^T, masked to -inf
        p   = exp(qk - LSE_i)                  (rebuilt, never stored)
        dV_j += p^T dO_i
        dp  = dO_i V_j^T
        ds  = p * (dp - D_i),  D = rowsum(dO * O)
        dQ_i += scale ds K_j ;  dK_j += scale ds^T Q_i
    """
    q, k, v, o, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, o, do))
    lse = np.asarray(lse, dtype=np.float64)
    N, d = q.shape
    scale = _as_scale(scale)
    causal = bool(mask_kind & MASK_CAUSAL)
    n_vis = N if kv_len is None else max(0, min(int(kv_len), N))
    q_blocks = list(partition(N, 64) if q_blocks is None else q_blocks)
    k_blocks = list(partition(N, 64) if k_blocks is None else k_blocks)
    D = (do * o).sum(axis=1)
    # Rows with no visible key: LSE = -inf; their p must be 0, not exp(+inf).
    base = np.where(np.isfinite(lse), lse, np.inf)
    dq = np.zeros((N, d))
    dk = np.zeros((N, d))
    dv = np.zeros((N, d))
    pairs = ([(i, j) for j in k_blocks for i in q_blocks] if key_outer
             else [(i, j) for i in q_blocks for j in k_blocks])
    for ri, cj in pairs:
        ri = np.asarray(ri, dtype=np.int64)
        cj = np.asarray(cj, dtype=np.int64)
        qk = (q[ri] @ k[cj].T) * scale
        qk = np.where(_visible(ri, cj, causal, n_vis), qk, -np.inf)
        p = np.exp(qk - base[ri, None])
        dv[cj] += p.T @ do[ri]
        dp = do[ri] @ v[cj].T
        ds = p * (dp - D[ri, None])
        dq[ri] += (ds @ k[cj]) * scale
        dk[cj] += (ds.T @ q[ri]) * scale
    return dq, dk, dv, D
