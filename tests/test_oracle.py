"""Pins for the CPU oracle: each check ties it to something other than itself.

Pins used (sources are cited by page title and section):

* the worked example of "FlashAttention算法详解：从IO瓶颈到Triton实现",
  section 一个小数值例子 (stored under tests/golden/),
* closed forms (Q = 0 gives a uniform softmax over the visible keys),
* invariants (rows of P sum to 1; V + c shifts O by c; any key-block
  partition and visiting order gives the same result, as the online-softmax
  section of the youngju.dev walkthrough, §6.2, states),
* reductions to independent library routines (scipy's logsumexp/softmax and
  PyTorch's CPU fp64 scaled_dot_product_attention),
* scalar brute force on tiny shapes.

The last test plants plausible mistakes into copies of the oracle's core and
checks that the pins catch every one of them.
"""
import importlib
import json
import math
import os

import numpy as np
import pytest

oracle_mod = importlib.import_module("oracle.attention_ref")
from oracle import (MASK_CAUSAL, MASK_KEY_PADDING, MASK_NONE, attention_ref,
                    brute_ref, online_attention_ref, online_softmax_stats,
                    partition, probabilities_ref)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")
MASKS = [MASK_NONE, MASK_CAUSAL, MASK_KEY_PADDING, MASK_CAUSAL | MASK_KEY_PADDING]


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _esum(exps):
    return math.fsum(math.exp(e) for e in exps)


def _rand(B, H, N, d, seed, qm=1.0):
    g = np.random.default_rng(seed)
    return (g.standard_normal((B, H, N, d)) * qm, g.standard_normal((B, H, N, d)),
            g.standard_normal((B, H, N, d)))


# --- the worked example -----------------------------------------------------

def test_worked_example_running_stats():
    ex = _golden()
    trace = online_softmax_stats(ex["logits"], ex["blocks"])
    (m1, l1), (m2, l2) = trace
    assert m1 == ex["after_block_1"]["m"]
    assert abs(l1 - _esum(ex["after_block_1"]["l_exponents"])) <= 1e-15
    assert m2 == ex["after_block_2"]["m"]
    assert abs(l2 - _esum(ex["after_block_2"]["l_exponents"])) <= 1e-15
    # The two pieces the page adds: old sum moved to the new max, new block.
    resc = l1 * math.exp(m1 - m2)
    assert abs(resc - _esum(ex["block_1_sum_rescaled_exponents"])) <= 1e-15
    assert abs((l2 - resc) - _esum(ex["block_2_contribution_exponents"])) <= 1e-15
    # One-shot: the same denominator with the max taken over the whole row.
    (m_all, l_all), = online_softmax_stats(ex["logits"], [[0, 1, 2, 3]])
    assert m_all == ex["one_shot_max"]
    assert abs(l_all - l2) <= 1e-15


@pytest.mark.parametrize("d,scale", [(4, 1.0), (64, 0.125)])
def test_worked_example_as_attention(d, scale):
    """Embed the row [1,2,3,0] as the logits of query 0; V = identity."""
    ex = _golden()
    logits = np.array(ex["logits"], dtype=np.float64)
    N = 4
    q = np.zeros((1, 1, N, d))
    k = np.zeros((1, 1, N, d))
    v = np.zeros((1, 1, N, d))
    q[0, 0, 0, 0] = 1.0 / scale
    k[0, 0, :, 0] = logits
    v[0, 0, :, :N] = np.eye(N)
    l2 = _esum(ex["after_block_2"]["l_exponents"])
    m2 = ex["after_block_2"]["m"]
    want_p = np.exp(logits - m2) / l2
    want_lse = m2 + math.log(l2)
    O, L = attention_ref(q, k, v, scale)
    assert np.max(np.abs(O[0, 0, 0, :N] - want_p)) <= 1e-15
    assert abs(L[0, 0, 0] - want_lse) <= 1e-15
    Oo, Lo = online_attention_ref(q[0, 0], k[0, 0], v[0, 0], scale,
                                  blocks=[np.array(b) for b in ex["blocks"]])
    assert np.max(np.abs(Oo[0, :N] - want_p)) <= 1e-15
    assert abs(Lo[0] - want_lse) <= 1e-15
    if d == 4:
        Ob, Lb = brute_ref(q, k, v, scale)
        assert np.max(np.abs(Ob[0, 0, 0, :N] - want_p)) <= 1e-15
        assert abs(Lb[0, 0, 0] - want_lse) <= 1e-15


# --- invariants ----------------------------------------------------------------

@pytest.mark.parametrize("mask", MASKS)
def test_rows_of_p_sum_to_one(mask):
    q, k, v = _rand(2, 2, 97, 16, seed=11)
    kv = np.array([40, 97], dtype=np.int32)
    ones = np.ones_like(v)
    O, _ = attention_ref(q, k, ones, 0.25, mask, kv)
    assert np.max(np.abs(O - 1.0)) <= 1e-12
    for b in range(2):
        P = probabilities_ref(q, k, 0.25, mask, kv, b=b, h=1)
        assert np.max(np.abs(P.sum(axis=1) - 1.0)) <= 1e-12
        assert (P >= 0).all()


@pytest.mark.parametrize("mask", MASKS)
def test_value_shift_equivariance(mask):
    q, k, v = _rand(1, 2, 70, 8, seed=12)
    kv = np.array([33], dtype=np.int32)
    O1, L1 = attention_ref(q, k, v, 0.3, mask, kv)
    O2, L2 = attention_ref(q, k, v + 2.5, 0.3, mask, kv)
    assert np.max(np.abs(O2 - (O1 + 2.5))) <= 1e-12
    assert np.array_equal(L1, L2)


@pytest.mark.parametrize("mask", MASKS)
def test_online_blocks_any_partition_and_order(mask):
    N, d = 131, 16
    q, k, v = _rand(1, 1, N, d, seed=13, qm=2.0)
    kv_len = 77
    O, L = attention_ref(q, k, v, 0.2, mask, np.array([kv_len], dtype=np.int32))
    rng = np.random.default_rng(5)
    for bs in (1, 2, 3, 7, 64, N):
        blocks = partition(N, bs)
        order = rng.permutation(len(blocks))
        blocks = [blocks[i] for i in order]
        Oo, Lo = online_attention_ref(q[0, 0], k[0, 0], v[0, 0], 0.2, mask,
                                      kv_len if mask & MASK_KEY_PADDING else None,
                                      blocks=blocks)
        assert np.max(np.abs(Oo - O[0, 0])) <= 1e-12, bs
        assert np.max(np.abs(Lo - L[0, 0])) <= 1e-12, bs
    # An irregular partition with shuffled members.
    perm = rng.permutation(N)
    cuts = np.sort(rng.choice(np.arange(1, N), 9, replace=False))
    blocks = np.split(perm, cuts)
    Oo, Lo = online_attention_ref(q[0, 0], k[0, 0], v[0, 0], 0.2, mask,
                                  kv_len if mask & MASK_KEY_PADDING else None, blocks=blocks)
    assert np.max(np.abs(Oo - O[0, 0])) <= 1e-12
    assert np.max(np.abs(Lo - L[0, 0])) <= 1e-12


# --- brute force on tiny shapes -------------------------------------------------

@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("N,d", [(1, 1), (3, 2), (5, 4), (8, 3)])
def test_brute_force_tiny(mask, N, d):
    q, k, v = _rand(2, 2, N, d, seed=100 + N * 10 + d)
    kv = np.array([0, max(1, N - 2)], dtype=np.int32)  # includes an empty batch entry
    for scale in (0.7, -1.3, 0.0):
        Ob, Lb = brute_ref(q, k, v, scale, mask, kv)
        O, L = attention_ref(q, k, v, scale, mask, kv, row_block=2)
        assert np.max(np.abs(O - Ob)) <= 1e-13
        fin = np.isfinite(Lb)
        assert np.array_equal(fin, np.isfinite(L))
        assert np.max(np.abs(L[fin] - Lb[fin]), initial=0.0) <= 1e-13


# --- closed forms ------------------------------------------------------------------

@pytest.mark.parametrize("mask", MASKS)
def test_q_zero_uniform_softmax(mask):
    """Q = 0: every logit is 0, P is uniform over the visible keys."""
    B, H, N, d = 2, 1, 1500, 8
    _, k, v = _rand(B, H, N, d, seed=14)
    q = np.zeros_like(k)
    kv = np.array([1, 1000], dtype=np.int32)
    O, L = attention_ref(q, k, v, 0.125, mask, kv, row_block=256)
    r = np.arange(N)
    for b in range(B):
        n_vis = kv[b] if mask & MASK_KEY_PADDING else N
        count = np.minimum(r + 1, n_vis) if mask & MASK_CAUSAL else np.full(N, n_vis)
        assert np.max(np.abs(L[b, 0] - np.log(count))) <= 1e-12
        csum = np.cumsum(v[b, 0], axis=0)               # prefix sums of V rows
        want = csum[count - 1] / count[:, None]
        assert np.max(np.abs(O[b, 0] - want)) <= 1e-12


def test_empty_rows_are_zero_with_minus_inf_lse():
    q, k, v = _rand(2, 1, 10, 4, seed=15)
    kv = np.array([0, 10], dtype=np.int32)
    O, L = attention_ref(q, k, v, 1.0, MASK_KEY_PADDING | MASK_CAUSAL, kv)
    assert np.all(O[0] == 0.0) and np.all(L[0] == -np.inf)
    assert np.all(np.isfinite(L[1]))


# --- reductions to library routines --------------------------------------------------

def test_unmasked_matches_scipy_softmax_and_logsumexp():
    from scipy.special import logsumexp, softmax
    q, k, v = _rand(1, 3, 200, 32, seed=16, qm=2.0)
    scale = 0.17677669
    O, L = attention_ref(q, k, v, scale)
    s = np.einsum("bhid,bhjd->bhij", q, k) * np.float64(np.float32(scale))
    assert np.max(np.abs(L - logsumexp(s, axis=-1))) <= 1e-12
    want = np.einsum("bhij,bhjd->bhid", softmax(s, axis=-1), v)
    assert np.max(np.abs(O - want)) <= 1e-12


@pytest.mark.parametrize("mask", MASKS)
def test_matches_torch_cpu_fp64_sdpa(mask):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    B, H, N, d = 2, 2, 150, 16
    q, k, v = _rand(B, H, N, d, seed=17)
    kv = np.array([150, 61], dtype=np.int32)
    scale = 0.25
    vis = np.ones((B, 1, N, N), dtype=bool)
    if mask & MASK_CAUSAL:
        vis &= np.tril(np.ones((N, N), dtype=bool))[None, None]
    if mask & MASK_KEY_PADDING:
        vis &= (np.arange(N)[None, :] < kv[:, None])[:, None, None, :]
    want = F.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(vis), scale=scale).numpy()
    O, _ = attention_ref(q, k, v, scale, mask, kv)
    assert np.max(np.abs(O - want)) <= 1e-12


# --- the oracle's own bookkeeping ---------------------------------------------------

def test_row_subsets_heads_and_blocking_agree():
    q, k, v = _rand(2, 3, 300, 8, seed=18)
    kv = np.array([300, 123], dtype=np.int32)
    mask = MASK_CAUSAL | MASK_KEY_PADDING
    O, L = attention_ref(q, k, v, 0.5, mask, kv)
    rows = np.array([0, 5, 64, 122, 123, 299])
    Os, Ls = attention_ref(q, k, v, 0.5, mask, kv, rows=rows, heads=[(1, 2), (0, 0)],
                           row_block=3)
    for b, h in [(1, 2), (0, 0)]:
        assert np.max(np.abs(Os[b, h] - O[b, h, rows])) <= 1e-13
        assert np.allclose(Ls[b, h], L[b, h, rows], rtol=0, atol=1e-13)
    assert np.isnan(Os[0, 1]).all()
    Ow, Lw = attention_ref(q, k, v, 0.5, mask, kv, workers=4, row_block=64)
    assert np.max(np.abs(Ow - O)) <= 1e-13


def test_scale_is_the_float32_value():
    q, k, v = _rand(1, 1, 20, 4, seed=19)
    s64 = 1.0 / math.sqrt(128.0)
    O1, _ = attention_ref(q, k, v, s64)
    O2, _ = attention_ref(q, k, v, float(np.float32(s64)))
    assert np.array_equal(O1, O2)


@pytest.mark.parametrize("mask", MASKS)
def test_forward_magnitudes(mask):
    """P |V| bounds |O| (equal when V >= 0); (sum_J |v|) / l bounds P |V|
    (P_rc = p_rc / l with p_rc <= 1); row-sum identity against probabilities_ref."""
    q, k, v = _rand(2, 2, 30, 6, seed=33)
    kv = np.array([0, 17], dtype=np.int32)
    O, L = attention_ref(q, k, v, 0.4, mask, kv)
    O2, L2, M = attention_ref(q, k, v, 0.4, mask, kv, magnitudes=True, row_block=7)
    assert np.array_equal(O, O2) or np.max(np.abs(O - O2)) <= 1e-13
    assert np.all(M["pv"] >= np.abs(O) - 1e-13)
    assert np.all(M["v_over_l"] >= M["pv"] - 1e-13)
    O3, _, M3 = attention_ref(q, k, np.abs(v), 0.4, mask, kv, magnitudes=True)
    assert np.max(np.abs(M3["pv"] - O3)) <= 1e-13
    for b in range(2):
        for h in range(2):
            P = probabilities_ref(q, k, 0.4, mask, kv, b, h)
            assert np.max(np.abs(M["pv"][b, h] - P @ np.abs(v[b, h]))) <= 1e-12


def test_rejects_bad_arguments():
    q, k, v = _rand(1, 1, 4, 2, seed=20)
    with pytest.raises(ValueError):
        attention_ref(q, k, v, 1.0, 4)
    with pytest.raises(ValueError):
        attention_ref(q, k, v, 1.0, MASK_KEY_PADDING, None)
    with pytest.raises(ValueError):
        attention_ref(q, k[:, :, :3], v, 1.0)


# --- planted mistakes must be caught by the pins ---------------------------------

MUTATIONS = {
    "scale dropped": ("s = (qh[rr] @ kh[:kmax].T) * scale", "s = (qh[rr] @ kh[:kmax].T)"),
    "causal mask off by one": ("cols[None, :] > rr[:, None]", "cols[None, :] >= rr[:, None]"),
    "causal mask flipped": ("cols[None, :] > rr[:, None]", "cols[None, :] < rr[:, None]"),
    "max not subtracted in LSE": ("lse[idx] = m[ok] + np.log(l)", "lse[idx] = np.log(l)"),
    "log base 2": ("np.log(l)", "np.log2(l)"),
    "no normalisation": ("/ l[:, None]", "/ 1.0"),
    "K not transposed (use K rows as columns)": ("kh[:kmax].T", "kh[:kmax].T[::-1]"),
    "V rows shifted": ("(p @ vh[:kmax])", "(p @ np.roll(vh[:kmax], 1, axis=0))"),
    "causal key range one short": ("int(rr.max()) + 1", "int(rr.max())"),
    "padding ignores kv_len": ("kmax = min(n_vis, int(rr.max()) + 1) if causal else n_vis",
                               "kmax = min(vh.shape[0], int(rr.max()) + 1) if causal else vh.shape[0]"),
    "masked logits leak into exp": ("p = np.exp(s[ok] - m[ok, None])",
                                    "p = np.exp(np.nan_to_num(s[ok], neginf=0.0) - m[ok, None])"),
    "LSE without the sum": ("lse[idx] = m[ok] + np.log(l)", "lse[idx] = m[ok]"),
}


def _pins_pass(mod) -> bool:
    """Run the pins above against a (possibly mutated) oracle module."""
    ref = mod.attention_ref
    try:
        ex = _golden()
        N, d = 4, 4
        q = np.zeros((1, 1, N, d)); k = np.zeros((1, 1, N, d)); v = np.zeros((1, 1, N, d))
        q[0, 0, 0, 0] = 2.0
        k[0, 0, :, 0] = np.array(ex["logits"], dtype=np.float64)
        v[0, 0, :, :N] = np.eye(N)
        l2 = _esum(ex["after_block_2"]["l_exponents"])
        O, L = ref(q, k, v, 0.5)
        if np.max(np.abs(O[0, 0, 0, :N] - np.exp(np.array(ex["logits"]) - 3.0) / l2)) > 1e-12:
            return False
        if abs(L[0, 0, 0] - (3.0 + math.log(l2))) > 1e-12:
            return False
        for mask in MASKS:
            qq, kk, vv = _rand(2, 1, 6, 3, seed=21)
            kv = np.array([0, 4], dtype=np.int32)
            Ob, Lb = brute_ref(qq, kk, vv, 0.6, mask, kv)
            Oa, La = ref(qq, kk, vv, 0.6, mask, kv)
            if np.max(np.abs(Oa - Ob)) > 1e-12:
                return False
            if not np.array_equal(np.isfinite(La), np.isfinite(Lb)):
                return False
            fin = np.isfinite(Lb)
            if np.max(np.abs(La[fin] - Lb[fin]), initial=0.0) > 1e-12:
                return False
        return True
    except Exception:
        return False


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name):
    import inspect
    src = inspect.getsource(oracle_mod)
    old, new = MUTATIONS[name]
    assert old in src, f"mutation anchor not found: {old!r}"
    ns = {"__name__": "mutated_oracle"}
    exec(compile(src.replace(old, new), "<mutated oracle>", "exec"), ns)

    class M:
        attention_ref = staticmethod(ns["attention_ref"])
    assert _pins_pass(oracle_mod), "pins must pass on the unmodified oracle"
    assert not _pins_pass(M), f"planted mistake not caught: {name}"


def test_oracle_is_independent_of_the_gpu_path():
    """The oracle imports neither the product package nor torch."""
    here = os.path.dirname(oracle_mod.__file__)
    for fn in os.listdir(here):
        if fn.endswith(".py"):
            text = open(os.path.join(here, fn)).read()
            assert "exact_attention_92_amd" not in text
            assert "import torch" not in text
