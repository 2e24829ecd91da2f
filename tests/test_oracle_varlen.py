"""Pins for the packed variable-length oracle.

* Packing B sequences of one common length gives the batched general
  oracle's result (a reshape), for every mask and window.
* Each sequence is attended on its own: changing another sequence's rows
  changes nothing here.
* A sequence without keys has O = 0 and LSE = -inf; one without queries
  writes nothing.
* Scalar brute force on a tiny packing with per-sequence positions written
  out (the queries sit at the last positions of the sequence's keys).
* Planted mistakes (global instead of per-sequence positions, a boundary
  off by one) fail these pins.
"""
import math

import numpy as np
import pytest

from oracle import MASK_CAUSAL, MASK_NONE, attention_general_ref, attention_varlen_ref


def _packed(lens_q, lens_k, H, d, seed):
    g = np.random.default_rng(seed)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    q = g.standard_normal((int(cu_q[-1]), H, d))
    k = g.standard_normal((int(cu_k[-1]), H, d))
    v = g.standard_normal((int(cu_k[-1]), H, d))
    return q, k, v, cu_q, cu_k


@pytest.mark.parametrize("mask", [MASK_NONE, MASK_CAUSAL])
@pytest.mark.parametrize("window", [-1, 0, 3])
def test_equal_lengths_are_the_batched_result(mask, window):
    B, H, nq, nk, d = 3, 2, 9, 14, 6
    q, k, v, cu_q, cu_k = _packed([nq] * B, [nk] * B, H, d, seed=11)
    O, L = attention_varlen_ref(q, k, v, cu_q, cu_k, 0.4, mask, window)
    qb = q.reshape(B, nq, H, d).transpose(0, 2, 1, 3)
    kb = k.reshape(B, nk, H, d).transpose(0, 2, 1, 3)
    vb = v.reshape(B, nk, H, d).transpose(0, 2, 1, 3)
    Ob, Lb = attention_general_ref(qb, kb, vb, 0.4, mask, window)
    np.testing.assert_array_equal(O, Ob.transpose(0, 2, 1, 3).reshape(B * nq, H, d))
    np.testing.assert_array_equal(L, Lb.transpose(1, 0, 2).reshape(H, B * nq))


def test_sequences_are_independent():
    q, k, v, cu_q, cu_k = _packed([5, 7, 4], [8, 3, 10], 2, 4, seed=12)
    O, L = attention_varlen_ref(q, k, v, cu_q, cu_k, 0.7, MASK_CAUSAL, 2)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[cu_q[1]:cu_q[2]] += 3.0
    k2[cu_k[1]:cu_k[2]] *= -2.0
    v2[cu_k[1]:cu_k[2]] += 1.0
    O2, L2 = attention_varlen_ref(q2, k2, v2, cu_q, cu_k, 0.7, MASK_CAUSAL, 2)
    for s in (0, 2):
        rows = slice(cu_q[s], cu_q[s + 1])
        np.testing.assert_array_equal(O2[rows], O[rows])
        np.testing.assert_array_equal(L2[:, rows], L[:, rows])
    assert not np.array_equal(O2[cu_q[1]:cu_q[2]], O[cu_q[1]:cu_q[2]])


def test_empty_sequences():
    q, k, v, cu_q, cu_k = _packed([3, 0, 4], [0, 5, 6], 2, 4, seed=13)
    O, L = attention_varlen_ref(q, k, v, cu_q, cu_k, 0.5, MASK_NONE)
    assert np.all(O[0:3] == 0.0) and np.all(L[:, 0:3] == -np.inf)   # no keys
    assert np.isfinite(O[3:]).all() and np.isfinite(L[:, 3:]).all()


def _brute(q, k, v, cu_q, cu_k, scale, causal, window):
    total_q, H, d = q.shape
    O = np.zeros((total_q, H, d))
    L = np.full((H, total_q), -np.inf)
    for b in range(len(cu_q) - 1):
        nq, nk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        for i in range(nq):
            pos = i + nk - nq                       # key position of this query in its sequence
            for h in range(H):
                logits = []
                for c in range(nk):
                    if causal and c > pos:
                        continue
                    if window >= 0 and c < pos - window:
                        continue
                    s = scale * sum(q[cu_q[b] + i, h, t] * k[cu_k[b] + c, h, t] for t in range(d))
                    logits.append((s, c))
                if not logits:
                    continue
                m = max(s for s, _ in logits)
                den = sum(math.exp(s - m) for s, _ in logits)
                for t in range(d):
                    O[cu_q[b] + i, h, t] = sum(math.exp(s - m) * v[cu_k[b] + c, h, t]
                                               for s, c in logits) / den
                L[h, cu_q[b] + i] = m + math.log(den)
    return O, L


@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 1), (False, 2)])
def test_brute_force_tiny(causal, window):
    q, k, v, cu_q, cu_k = _packed([3, 1, 4], [5, 2, 4], 2, 3, seed=14)
    mask = MASK_CAUSAL if causal else MASK_NONE
    O, L = attention_varlen_ref(q, k, v, cu_q, cu_k, 0.9, mask, window)
    Ob, Lb = _brute(q, k, v, cu_q, cu_k, float(np.float32(0.9)), causal, window)
    assert np.max(np.abs(O - Ob)) <= 1e-12
    assert np.array_equal(np.isfinite(L), np.isfinite(Lb))
    assert np.max(np.abs(L[np.isfinite(L)] - Lb[np.isfinite(Lb)]), initial=0.0) <= 1e-12


MUTATIONS = {
    "key slice one row short": ("qs, qe, ks, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), "
                                "int(cu_k[b + 1])",
                                "qs, qe, ks, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), "
                                "int(cu_k[b + 1]) - 1"),
    "keys of the query boundaries": ("kb = k[ks:ke].transpose(1, 0, 2)[None]",
                                     "kb = k[qs:qe].transpose(1, 0, 2)[None]"),
    "empty-key rows left unwritten": ("            O[qs:qe] = 0.0\n", "            pass\n"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name):
    import importlib
    import inspect
    mod = importlib.import_module("oracle.attention_ref")
    src = inspect.getsource(mod)
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, name
    ns = {"__name__": "mutated"}
    exec(compile(src.replace(old, new), "<mutated>", "exec"), ns)
    q, k, v, cu_q, cu_k = _packed([3, 1, 4, 2], [5, 0, 4, 2], 2, 3, seed=15)
    caught = False
    for causal, window in ((False, -1), (True, -1), (True, 1)):
        mask = MASK_CAUSAL if causal else MASK_NONE
        Ob, Lb = _brute(q, k, v, cu_q, cu_k, float(np.float32(0.9)), causal, window)
        try:
            O, L = ns["attention_varlen_ref"](q, k, v, cu_q, cu_k, 0.9, mask, window)
        except Exception:
            caught = True
            continue
        if not (np.nanmax(np.abs(O - Ob), initial=0.0) <= 1e-12) or np.isnan(O).any():
            caught = True
    assert caught, name
