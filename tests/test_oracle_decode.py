"""Pins for the paged-decode oracle.

* Against the forward oracle (pinned in test_oracle.py): with a cache laid
  out contiguously, decode of the newest token equals the last row of causal
  self-attention over the cached tokens ("FlashAttention 完整解析" §7: the
  block table only changes where keys and values are read from).
* Block placement does not matter: permuting the physical blocks and the
  table together gives bit-identical results.
* Closed form: q = 0 gives the mean of the request's V rows and LSE = ln n.
* Scalar brute force on tiny shapes; n = 0 gives O = 0 and LSE = -inf.
"""
import importlib
import math

import numpy as np
import pytest

from fa_inputs import bf16_bits_to_f32, make_paged_decode
from oracle import MASK_CAUSAL, attention_ref
from oracle.paged_decode_ref import gather_paged, paged_decode_ref

dec_mod = importlib.import_module("oracle.paged_decode_ref")


def _f64(a):
    return bf16_bits_to_f32(a).astype(np.float64)


def _batch(seed=1, B=3, H=2, d=16, bs=8, lens=(5, 40)):
    x = make_paged_decode(B, H, d, bs, lens, seed)
    return (_f64(x["q"]), _f64(x["k_pool"]), _f64(x["v_pool"]), x["block_tables"],
            x["seq_lens"])


def test_generator_recipe():
    x = make_paged_decode(5, 2, 16, 8, (1, 60), seed=3, spare=4)
    lens, tab = x["seq_lens"], x["block_tables"]
    nblk = (lens + 7) // 8
    used = np.concatenate([tab[b, :nblk[b]] for b in range(5)])
    assert len(set(used.tolist())) == len(used)                  # no block shared
    assert x["k_pool"].shape[0] == len(used) + 4                  # plus the spares
    assert all(np.all(tab[b, nblk[b]:] == -1) for b in range(5))
    y = make_paged_decode(5, 2, 16, 8, (1, 60), seed=3, spare=4)
    assert all(np.array_equal(x[k], y[k]) for k in x)


@pytest.mark.parametrize("seed", [1, 2])
def test_equals_last_row_of_causal_attention(seed):
    q, kp, vp, tab, lens = _batch(seed)
    scale = 0.3
    O, L = paged_decode_ref(q, kp, vp, tab, lens, scale)
    for b in range(q.shape[0]):
        n = int(lens[b])
        for h in range(q.shape[1]):
            K = gather_paged(kp, tab[b], n, h)
            V = gather_paged(vp, tab[b], n, h)
            Q = np.zeros_like(K)
            Q[-1] = q[b, h]
            Oc, Lc = attention_ref(Q[None, None], K[None, None], V[None, None], scale,
                                   MASK_CAUSAL, rows=[n - 1])
            assert np.max(np.abs(O[b, h] - Oc[0, 0, 0])) <= 1e-13
            assert abs(L[b, h] - Lc[0, 0, 0]) <= 1e-13


def test_contiguous_cache_against_forward_oracle_directly():
    """Identity block table over one request: the pool is the cache itself."""
    g = np.random.default_rng(4)
    H, d, bs, n = 2, 8, 4, 13
    nb = (n + bs - 1) // bs
    K = g.standard_normal((H, nb * bs, d))
    V = g.standard_normal((H, nb * bs, d))
    Qn = g.standard_normal((H, d))
    kp = K.reshape(H, nb, bs, d).transpose(1, 0, 2, 3)
    vp = V.reshape(H, nb, bs, d).transpose(1, 0, 2, 3)
    tab = np.arange(nb, dtype=np.int32)[None]
    O, L = paged_decode_ref(Qn[None], kp, vp, tab, np.array([n]), 0.5)
    Q = np.zeros((1, H, n, d))
    Q[0, :, n - 1] = Qn
    Oc, Lc = attention_ref(Q, K[None, :, :n], V[None, :, :n], 0.5, MASK_CAUSAL, rows=[n - 1])
    assert np.max(np.abs(O[0] - Oc[0, :, 0])) <= 1e-13
    assert np.max(np.abs(L[0] - Lc[0, :, 0])) <= 1e-13


def test_block_placement_does_not_matter():
    q, kp, vp, tab, lens = _batch(5)
    O, L = paged_decode_ref(q, kp, vp, tab, lens, 0.25)
    perm = np.random.default_rng(0).permutation(kp.shape[0])
    inv = np.argsort(perm)
    tab2 = np.where(tab >= 0, inv[np.maximum(tab, 0)], -1).astype(np.int32)
    O2, L2 = paged_decode_ref(q, kp[perm], vp[perm], tab2, lens, 0.25)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_q_zero_closed_form_and_empty_request():
    q, kp, vp, tab, lens = _batch(6)
    lens = lens.copy()
    lens[1] = 0
    O, L = paged_decode_ref(np.zeros_like(q), kp, vp, tab, lens, 0.7)
    for b in range(q.shape[0]):
        n = int(lens[b])
        for h in range(q.shape[1]):
            if n == 0:
                assert np.all(O[b, h] == 0) and L[b, h] == -np.inf
                continue
            V = gather_paged(vp, tab[b], n, h)
            assert np.max(np.abs(O[b, h] - V.mean(axis=0))) <= 1e-13
            assert abs(L[b, h] - math.log(n)) <= 1e-13


def test_brute_force_tiny():
    q, kp, vp, tab, lens = _batch(7, B=2, H=2, d=3, bs=2, lens=(1, 7))
    O, L = paged_decode_ref(q, kp, vp, tab, lens, 0.9)
    for b in range(2):
        for h in range(2):
            n = int(lens[b])
            toks = [(int(tab[b, t // 2]), t % 2) for t in range(n)]
            sc = float(np.float32(0.9))          # the float32 scale a kernel receives
            s = [sc * math.fsum(q[b, h, i] * kp[p, h, o, i] for i in range(3)) for p, o in toks]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            den = math.fsum(e)
            for i in range(3):
                want = math.fsum(e[t] * vp[toks[t][0], h, toks[t][1], i] for t in range(n)) / den
                assert abs(O[b, h, i] - want) <= 1e-13
            assert abs(L[b, h] - (m + math.log(den))) <= 1e-13


MUTATIONS = {
    "slot taken from the wrong block": ("parts = [pool[int(table_row[j]), h] for j in range(nb)]",
                                        "parts = [pool[j, h] for j in range(nb)]"),
    "one token short": ("np.concatenate(parts, axis=0)[:n]", "np.concatenate(parts, axis=0)[:n - 1]"),
    "scale dropped": ("s = (K @ q[b, h]) * scale", "s = (K @ q[b, h])"),
    "no normalisation": ("O[b, h] = (e @ V) / e.sum()", "O[b, h] = (e @ V)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name):
    import inspect
    src = inspect.getsource(dec_mod)
    old, new = MUTATIONS[name]
    assert src.count(old) == 1
    ns = {"__name__": "mutated_decode"}
    exec(compile(src.replace(old, new), "<mutated>", "exec"), ns)
    q, kp, vp, tab, lens = _batch(8)
    O, L = ns["paged_decode_ref"](q, kp, vp, tab, lens, 0.3)
    b, h = 0, 0
    n = int(lens[b])
    K = gather_paged(kp, tab[b], n, h)
    V = gather_paged(vp, tab[b], n, h)
    Q = np.zeros_like(K)
    Q[-1] = q[b, h]
    Oc, Lc = attention_ref(Q[None, None], K[None, None], V[None, None], 0.3, MASK_CAUSAL,
                           rows=[n - 1])
    caught = np.max(np.abs(O[b, h] - Oc[0, 0, 0])) > 1e-9 or abs(L[b, h] - Lc[0, 0, 0]) > 1e-9
    assert caught, name
