"""CPU oracle for the exact scaled-dot-product attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the package's smoke check and the
bench's CPU-baseline leg use it.  It shares no code with the HIP kernels.

Sources (web pages; cited by title and section):

* [G]  "FlashAttention算法详解：从IO瓶颈到Triton实现" (gentlecold.top)
* [Y]  FlashAttention paper walkthrough, flash_attention.zh (youngju.dev)
* [F]  "FlashAttention 完整解析：从原理到 CUDA/Triton 实现" (freezetheflame.cc)

What is computed (the plain definition, fp64 throughout):

    O = softmax(scale * Q K^T + M) V                      [G] 先说结论 (the equation)
    LSE_r = m_r + ln l_r                                   [G] Backward为什么更复杂

for every batch entry b and head h, with the additive mask M equal to 0 on
the visible key set J_r of query row r and -inf elsewhere:

    J_r = { c : c < N,
                c <= r          if causal           [G] Causal Mask怎么处理
                c < kv_len[b]   if key padding }    [G] FlashAttention Forward流程 ("padding")

The softmax is the max-subtracted ("safe") form of [G] Online Softmax and
[Y] §6.1.  The oracle materialises S and P, one block of query rows at a
time (the full N x N never fits at N = 65536); the row blocking only bounds
memory and does not change any row's arithmetic.  The two products are
plain BLAS matrix products.

Readings where the pages are silent (each is also listed in the design
notes):

* A row with no visible key (kv_len = 0) has O_r = 0 and LSE_r = -inf.
* ``scale`` is used as the float32 value a kernel receives, widened to
  float64.
* LSE is in natural-log units of the scaled logits.

``online_attention_ref`` follows the blocked online-softmax recurrence of
[G] Online Softmax / FlashAttention Forward流程 and [Y] §6.2 in fp64, with an
arbitrary key-block partition and visiting order; it exists to pin the
recurrence (the worked example, block-order independence), not for parity.
``brute_ref`` is the same definition as scalar Python loops with
``math.exp``/``math.fsum`` for tiny shapes.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from typing import Iterable, List, Optional, Sequence

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_KEY_PADDING = 2


def _as_scale(scale: float) -> float:
    return float(np.float32(scale))


def _kv_len(mask_kind: int, kv_lens, b: int, N: int) -> int:
    if mask_kind & MASK_KEY_PADDING:
        return max(0, min(int(kv_lens[b]), N))
    return N


def _head_ref(qh, kh, vh, scale, causal, n_vis, rows, row_block, mags=None):
    """Definition of O and LSE for one (b, h) over the query rows ``rows``.
    With ``mags`` (a dict), also P |V| and (sum over visible keys of |V|) / l."""
    d = vh.shape[1]
    out = np.zeros((len(rows), d), dtype=np.float64)
    lse = np.full(len(rows), -np.inf, dtype=np.float64)
    if mags is not None:
        mags["pv"] = np.zeros((len(rows), d))
        mags["v_over_l"] = np.zeros((len(rows), d))
    for start in range(0, len(rows), row_block):
        rr = rows[start:start + row_block]
        kmax = min(n_vis, int(rr.max()) + 1) if causal else n_vis
        if kmax <= 0:
            continue
        # S = scale * Q K^T on the keys that can be visible to this block.
        s = (qh[rr] @ kh[:kmax].T) * scale
        if causal:
            cols = np.arange(kmax)
            s[cols[None, :] > rr[:, None]] = -np.inf
        m = s.max(axis=1)
        ok = np.isfinite(m)                      # rows with >= 1 visible key
        p = np.exp(s[ok] - m[ok, None])          # exp(S - rowmax), masked -> 0
        l = p.sum(axis=1)
        idx = start + np.nonzero(ok)[0]
        out[idx] = (p @ vh[:kmax]) / l[:, None]  # P V with P = p / l
        lse[idx] = m[ok] + np.log(l)
        if mags is not None:
            av = np.abs(vh[:kmax])
            mags["pv"][idx] = (p @ av) / l[:, None]
            mags["v_over_l"][idx] = (np.isfinite(s[ok]).astype(np.float64) @ av) / l[:, None]
    return out, lse


def attention_ref(q, k, v, scale, mask_kind=MASK_NONE, kv_lens=None,
                  rows: Optional[Sequence[int]] = None, heads=None,
                  row_block: int = 512, workers: int = 1, magnitudes: bool = False):
    """fp64 O and LSE of exact attention.

    q, k, v: float64 arrays ``[B, H, N, d]`` (callers widen the generated
    bf16/fp32 data exactly).  ``rows``: optional sorted query-row indices to
    compute (default: all).  ``heads``: optional list of (b, h) pairs
    (default: all).  Returns ``O [B, H, R, d]`` and ``LSE [B, H, R]``; rows
    of heads not requested are left NaN.

    ``magnitudes=True`` appends a dict with, per output element, ``pv`` =
    (P |V|)_rt and ``v_over_l`` = (sum over the visible keys of |v_ct|) / l_r,
    with l_r the max-subtracted row sum (at least 1).  They bound how far
    per-probability rounding errors (relative and absolute) can move O; they
    are for tolerances only.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    if k.shape != (B, H, N, d) or v.shape != (B, H, N, d):
        raise ValueError("q, k, v must share the shape [B, H, N, d]")
    if mask_kind & ~(MASK_CAUSAL | MASK_KEY_PADDING):
        raise ValueError(f"unknown mask bits in {mask_kind}")
    if (mask_kind & MASK_KEY_PADDING) and kv_lens is None:
        raise ValueError("key padding needs kv_lens")
    scale = _as_scale(scale)
    causal = bool(mask_kind & MASK_CAUSAL)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    units = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    O = np.full((B, H, len(rows), d), np.nan)
    L = np.full((B, H, len(rows)), np.nan)
    M = ({"pv": np.full(O.shape, np.nan), "v_over_l": np.full(O.shape, np.nan)}
         if magnitudes else None)

    def run(unit):
        b, h = unit
        n_vis = _kv_len(mask_kind, kv_lens, b, N)
        mags = {} if magnitudes else None
        O[b, h], L[b, h] = _head_ref(q[b, h], k[b, h], v[b, h], scale, causal,
                                     n_vis, rows, row_block, mags)
        if magnitudes:
            for name in M:
                M[name][b, h] = mags[name]

    if workers <= 1 or len(units) == 1:
        for u in units:
            run(u)
    else:
        # Parallel over independent heads only; each head's arithmetic is the
        # same as in the serial loop.  BLAS is held to one thread per worker.
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
            list(ex.map(run, units))
    if magnitudes:
        return O, L, M
    return O, L


def probabilities_ref(q, k, scale, mask_kind=MASK_NONE, kv_lens=None, b=0, h=0):
    """The full fp64 probability matrix P of one head (small N only)."""
    q = np.asarray(q, dtype=np.float64)[b, h]
    k = np.asarray(k, dtype=np.float64)[b, h]
    N = q.shape[0]
    s = (q @ k.T) * _as_scale(scale)
    vis = np.ones((N, N), dtype=bool)
    if mask_kind & MASK_CAUSAL:
        vis &= np.arange(N)[None, :] <= np.arange(N)[:, None]
    if mask_kind & MASK_KEY_PADDING:
        vis &= np.arange(N)[None, :] < _kv_len(mask_kind, kv_lens, b, N)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    P = np.zeros_like(s)
    ok = np.isfinite(m)
    e = np.exp(s[ok] - m[ok, None])
    P[ok] = e / e.sum(axis=1, keepdims=True)
    return P


# ---------------------------------------------------------------------------
# The online (blocked) recurrence, in the pages' notation.
# ---------------------------------------------------------------------------

def online_softmax_stats(x: Sequence[float], blocks: Sequence[Sequence[int]]):
    """Running (m, l) of one logit row, visiting key blocks in the given order.

    Per block:  m_new = max(m, max(block));
                l_new = l * exp(m - m_new) + sum_{j in block} exp(x_j - m_new)
    ([G] Online Softmax; [Y] §6.2).  Returns the list of (m, l) after each
    block, starting from m = -inf, l = 0.
    """
    m, l = -math.inf, 0.0
    trace = []
    for blk in blocks:
        vals = [float(x[j]) for j in blk]
        m_new = max([m] + vals)
        if m_new == -math.inf:
            trace.append((m, l))
            continue
        alpha = math.exp(m - m_new) if m != -math.inf else 0.0
        l = l * alpha + math.fsum(math.exp(t - m_new) for t in vals)
        m = m_new
        trace.append((m, l))
    return trace


def partition(N: int, block: int) -> List[np.ndarray]:
    """Split key indices 0..N-1 into consecutive blocks of ``block`` keys."""
    return [np.arange(s, min(N, s + block)) for s in range(0, N, block)]


def online_attention_ref(q, k, v, scale, mask_kind=MASK_NONE, kv_len=None,
                         blocks: Optional[Iterable[np.ndarray]] = None):
    """One head's O and LSE by the blocked online-softmax loop, in fp64.

    q, k, v: ``[N, d]`` float64.  ``blocks``: key-index blocks in visiting
    order (any partition of 0..N-1, any order).  Every query row is carried
    through the same loop ([G] FlashAttention Forward流程):

        qk    = scale * Q K_j^T, masked to -inf
        m_new = max(m, rowmax(qk))
        p     = exp(qk - m_new);  alpha = exp(m - m_new)
        acc   = alpha * acc + p V_j;  l = alpha * l + rowsum(p);  m = m_new
        O = acc / l;  LSE = m + ln l

    Rows whose running max is still -inf use 0 in place of m_new, so their p
    is 0 (masked) and alpha is irrelevant (acc and l are still 0).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    scale = _as_scale(scale)
    if blocks is None:
        blocks = partition(N, 64)
    n_vis = N if kv_len is None else max(0, min(int(kv_len), N))
    rows = np.arange(N)
    m = np.full(N, -np.inf)
    l = np.zeros(N)
    acc = np.zeros((N, d))
    for cols in blocks:
        cols = np.asarray(cols, dtype=np.int64)
        qk = (q @ k[cols].T) * scale
        vis = np.ones(qk.shape, dtype=bool)
        if mask_kind & MASK_CAUSAL:
            vis &= cols[None, :] <= rows[:, None]
        if mask_kind & MASK_KEY_PADDING:
            vis &= cols[None, :] < n_vis
        qk = np.where(vis, qk, -np.inf)
        m_new = np.maximum(m, qk.max(axis=1))
        base = np.where(np.isfinite(m_new), m_new, 0.0)
        p = np.exp(qk - base[:, None])
        alpha = np.where(np.isfinite(m), np.exp(m - base), 0.0)
        acc = alpha[:, None] * acc + p @ v[cols]
        l = alpha * l + p.sum(axis=1)
        m = m_new
    out = np.zeros((N, d))
    lse = np.full(N, -np.inf)
    ok = l > 0
    out[ok] = acc[ok] / l[ok, None]
    lse[ok] = m[ok] + np.log(l[ok])
    return out, lse


# ---------------------------------------------------------------------------
# Scalar brute force for tiny shapes.
# ---------------------------------------------------------------------------

def brute_ref(q, k, v, scale, mask_kind=MASK_NONE, kv_lens=None):
    """Pure-Python loops of the definition (math.exp, math.fsum); tiny N only."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    scale = _as_scale(scale)
    O = np.zeros((B, H, N, d))
    L = np.full((B, H, N), -np.inf)
    for b in range(B):
        n_vis = _kv_len(mask_kind, kv_lens, b, N)
        for h in range(H):
            for r in range(N):
                J = [c for c in range(N)
                     if c < n_vis and (not (mask_kind & MASK_CAUSAL) or c <= r)]
                if not J:
                    continue
                s = {c: scale * math.fsum(float(q[b, h, r, t]) * float(k[b, h, c, t])
                                          for t in range(d)) for c in J}
                mx = max(s.values())
                e = {c: math.exp(s[c] - mx) for c in J}
                den = math.fsum(e.values())
                for t in range(d):
                    O[b, h, r, t] = math.fsum(e[c] * float(v[b, h, c, t]) for c in J) / den
                L[b, h, r] = mx + math.log(den)
    return O, L


# ---------------------------------------------------------------------------
# General masks: N_q != N_k, sliding window.
# ---------------------------------------------------------------------------

def visible_general(Nq: int, Nk: int, causal: bool, window_left: int, n_vis: int,
                    rows=None):
    """Boolean [Nq, Nk] visibility for the general forward (only the query
    rows ``rows`` when given: [len(rows), Nk]).

    Query r sits at key position a_r = r + (Nk - Nq) (the queries are the last
    Nq positions of the key sequence).  Key c is visible to query r iff
    c < n_vis, and c <= a_r when causal, and c >= a_r - window_left when
    window_left >= 0 (a window of window_left keys before the query's own
    position).
    """
    rr = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    r = rr[:, None] + (Nk - Nq)
    c = np.arange(Nk)[None, :]
    vis = c < n_vis
    if causal:
        vis = vis & (c <= r)
    if window_left >= 0:
        vis = vis & (c >= r - window_left)
    return np.broadcast_to(vis, (len(rr), Nk))


def attention_general_ref(q, k, v, scale, mask_kind=MASK_NONE, window_left: int = -1,
                          kv_lens=None, magnitudes: bool = False, rows=None):
    """fp64 O [B, H, Nq, d] and LSE [B, H, Nq] with N_q != N_k allowed and an
    optional sliding window (see visible_general); the same definition as
    attention_ref otherwise (max-subtracted softmax over the visible keys;
    a row with no visible key has O = 0, LSE = -inf).  ``magnitudes=True``
    appends P |V| [B, H, Nq, d] (for tolerances).  ``rows``: optional query
    row indices; then only those rows are computed and the outputs are
    [B, H, R, ...] in that order."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape:
        raise ValueError("k, v must be [B, H, Nk, d] with q's B, H, d")
    if mask_kind & ~(MASK_CAUSAL | MASK_KEY_PADDING):
        raise ValueError(f"unknown mask bits in {mask_kind}")
    if (mask_kind & MASK_KEY_PADDING) and kv_lens is None:
        raise ValueError("key padding needs kv_lens")
    scale = _as_scale(scale)
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows)
    O = np.zeros((B, H, R, d))
    L = np.full((B, H, R), -np.inf)
    M = np.zeros((B, H, R, d))
    for b in range(B):
        n_vis = _kv_len(mask_kind, kv_lens, b, Nk)
        vis = visible_general(Nq, Nk, bool(mask_kind & MASK_CAUSAL), window_left, n_vis, rows)
        ok = vis.any(axis=1)
        for h in range(H):
            s = np.where(vis, (q[b, h, rows] @ k[b, h].T) * scale, -np.inf)
            m = s[ok].max(axis=1)
            e = np.exp(s[ok] - m[:, None])
            l = e.sum(axis=1)
            O[b, h, ok] = (e @ v[b, h]) / l[:, None]
            L[b, h, ok] = m + np.log(l)
            M[b, h, ok] = (e @ np.abs(v[b, h])) / l[:, None]
    if magnitudes:
        return O, L, M
    return O, L


def attention_varlen_ref(q, k, v, cu_q, cu_k, scale, mask_kind=MASK_NONE,
                         window_left: int = -1, magnitudes: bool = False):
    """fp64 attention over packed variable-length sequences.

    q: [total_q, H, d]; k, v: [total_k, H, d]; cu_q, cu_k: int [B + 1]
    sequence boundaries.  Sequence b is the query rows cu_q[b]:cu_q[b+1]
    attending to the key rows cu_k[b]:cu_k[b+1] on its own, with the
    conventions of attention_general_ref (queries at the last positions of
    the sequence's keys; causal and window act within the sequence).
    Returns O [total_q, H, d] and LSE [H, total_q] (and P |V| [total_q, H, d]
    with ``magnitudes``).  Rows not covered by any sequence stay NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    total_q, H, d = q.shape
    O = np.full((total_q, H, d), np.nan)
    L = np.full((H, total_q), np.nan)
    M = np.full((total_q, H, d), np.nan)
    if mask_kind & ~MASK_CAUSAL:
        raise ValueError("packed sequences take their key lengths from cu_k: causal bit only")
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if qe <= qs:
            continue
        if ke <= ks:                       # no keys: every row is empty
            O[qs:qe] = 0.0
            L[:, qs:qe] = -np.inf
            M[qs:qe] = 0.0
            continue
        qb = q[qs:qe].transpose(1, 0, 2)[None]     # [1, H, n_q, d]
        kb = k[ks:ke].transpose(1, 0, 2)[None]
        vb = v[ks:ke].transpose(1, 0, 2)[None]
        Ob, Lb, Mb = attention_general_ref(qb, kb, vb, scale, mask_kind, window_left,
                                           magnitudes=True)
        O[qs:qe] = Ob[0].transpose(1, 0, 2)
        L[:, qs:qe] = Lb[0]
        M[qs:qe] = Mb[0].transpose(1, 0, 2)
    if magnitudes:
        return O, L, M
    return O, L
