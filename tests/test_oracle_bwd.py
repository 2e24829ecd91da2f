"""Pins for the backward oracle: each ties it to something other than itself.

Pins used (sources are cited by page title and section):

* finite differences of the scalar sum(dO * O) through the forward oracle
  (itself pinned in test_oracle.py): the gradients the backward equations of
  "FlashAttention算法详解：从IO瓶颈到Triton实现" (section Backward为什么更复杂)
  produce must be the derivatives of the forward's output,
* reduction to an independent library: PyTorch CPU fp64 autograd through
  scaled_dot_product_attention (the math backend the youngju.dev
  walkthrough lists in §11),
* closed forms for Q = 0 (uniform probabilities over the visible keys),
* invariants: the rows of dS sum to zero (so the key gradients sum to zero),
  the value gradients sum to the summed upstream gradient, and shifting
  every key (or every value) by one vector leaves dQ and dK unchanged,
* the identity rowsum(dP * P) = rowsum(dO * O) against the forward oracle,
* the block scan with probabilities rebuilt from the saved LSE ([G] section
  Backward为什么更复杂, the flowchart; youngju.dev §7.2) over any partition
  and visiting order.

The last test plants plausible mistakes into copies of the oracle and checks
that the pins catch every one of them.
"""
import importlib

import numpy as np
import pytest

from oracle import (MASK_CAUSAL, MASK_KEY_PADDING, MASK_NONE, attention_bwd_ref,
                    attention_ref, blocked_attention_bwd_ref, partition)

bwd_mod = importlib.import_module("oracle.attention_bwd_ref")

MASKS = [MASK_NONE, MASK_CAUSAL, MASK_KEY_PADDING, MASK_CAUSAL | MASK_KEY_PADDING]


def _rand(B, H, N, d, seed, qm=1.0):
    g = np.random.default_rng(seed)
    return tuple(g.standard_normal((B, H, N, d)) * (qm if i == 0 else 1.0) for i in range(4))


def _fd_grads(q, k, v, do, scale, mask, kv, h=1e-6):
    """Central differences of L = sum(dO * O(Q, K, V)) via the forward oracle."""
    def loss(qq, kk, vv):
        O, _ = attention_ref(qq, kk, vv, scale, mask, kv)
        return float(np.sum(do * O))
    out = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(q)
        for idx in np.ndindex(q.shape):
            plus = [t.copy() for t in base]
            minus = [t.copy() for t in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        out.append(g)
    return out


# --- derivatives of the forward ------------------------------------------------

@pytest.mark.parametrize("mask", MASKS)
def test_gradients_are_finite_difference_derivatives(mask):
    q, k, v, do = _rand(2, 1, 6, 3, seed=40 + mask)
    kv = np.array([0, 4], dtype=np.int32)
    scale = 0.7
    dQ, dK, dV, _ = attention_bwd_ref(q, k, v, do, scale, mask, kv)
    for got, want, name in zip((dQ, dK, dV), _fd_grads(q, k, v, do, scale, mask, kv), "QKV"):
        assert np.max(np.abs(got - want)) <= 2e-7, f"d{name} mask={mask}"


def test_finite_differences_odd_shape_and_scale():
    q, k, v, do = _rand(1, 2, 7, 4, seed=3, qm=2.0)
    scale = float(np.float32(0.37))
    dQ, dK, dV, _ = attention_bwd_ref(q, k, v, do, scale, MASK_CAUSAL)
    for got, want in zip((dQ, dK, dV), _fd_grads(q, k, v, do, scale, MASK_CAUSAL, None)):
        assert np.max(np.abs(got - want)) <= 2e-7


# --- an independent library ------------------------------------------------------

@pytest.mark.parametrize("mask", MASKS)
def test_matches_torch_cpu_fp64_autograd(mask):
    torch = pytest.importorskip("torch")
    B, H, N, d = 3, 2, 37, 16
    q, k, v, do = _rand(B, H, N, d, seed=7 + mask, qm=1.5)
    kv = np.array([37, 1, 20], dtype=np.int32)
    scale = 0.25
    vis = np.ones((B, 1, N, N), dtype=bool)
    if mask & MASK_CAUSAL:
        vis &= np.tril(np.ones((N, N), dtype=bool))[None, None]
    if mask & MASK_KEY_PADDING:
        vis &= (np.arange(N)[None, :] < kv[:, None])[:, None, None, :]
    tq, tk, tv = (torch.tensor(t, dtype=torch.float64, requires_grad=True) for t in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(vis), scale=scale)
    out.backward(torch.tensor(do))
    dQ, dK, dV, _ = attention_bwd_ref(q, k, v, do, scale, mask, kv)
    for got, t, name in zip((dQ, dK, dV), (tq, tk, tv), "QKV"):
        assert np.max(np.abs(got - t.grad.numpy())) <= 1e-12, f"d{name} mask={mask}"


# --- closed forms and invariants -----------------------------------------------------

def _vis_sets(N, mask, kvl):
    return [[c for c in range(N) if c < kvl and (not (mask & MASK_CAUSAL) or c <= r)]
            for r in range(N)]


@pytest.mark.parametrize("mask", MASKS)
def test_q_zero_closed_forms(mask):
    """Q = 0: P_r is uniform over J_r.  Then dK = 0 exactly,
    dV_c = sum_{r : c in J_r} dO_r / |J_r|, and
    dQ_r = scale / |J_r| * sum_{c in J_r} (dO_r . (v_c - mean_J v)) k_c."""
    B, H, N, d = 2, 2, 19, 5
    _, k, v, do = _rand(B, H, N, d, seed=11)
    q = np.zeros_like(k)
    kv = np.array([13, 0], dtype=np.int32)
    scale = 0.5
    dQ, dK, dV, _ = attention_bwd_ref(q, k, v, do, scale, mask, kv)
    assert np.all(dK == 0.0)
    for b in range(B):
        kvl = int(kv[b]) if mask & MASK_KEY_PADDING else N
        J = _vis_sets(N, mask, kvl)
        for h in range(H):
            wv = np.zeros((N, d))
            wq = np.zeros((N, d))
            for r in range(N):
                if not J[r]:
                    continue
                n = len(J[r])
                wv[J[r]] += do[b, h, r] / n
                vbar = v[b, h, J[r]].mean(axis=0)
                coef = (v[b, h, J[r]] - vbar) @ do[b, h, r]
                wq[r] = scale / n * (coef @ k[b, h, J[r]])
            assert np.max(np.abs(dV[b, h] - wv)) <= 1e-13
            assert np.max(np.abs(dQ[b, h] - wq)) <= 1e-13


@pytest.mark.parametrize("mask", MASKS)
def test_key_and_value_gradient_sums(mask):
    """Rows of dS sum to zero, so sum_c dK_c = 0; rows of P sum to one over
    J_r, so sum_c dV_c = sum of dO over the rows that see a key."""
    B, H, N, d = 2, 3, 50, 8
    q, k, v, do = _rand(B, H, N, d, seed=12, qm=2.0)
    kv = np.array([31, 50], dtype=np.int32)
    dQ, dK, dV, _ = attention_bwd_ref(q, k, v, do, 0.3, mask, kv, row_block=16)
    scale_ref = np.abs(dK).sum(axis=2)
    assert np.all(np.abs(dK.sum(axis=2)) <= 1e-12 * np.maximum(scale_ref, 1.0))
    for b in range(B):
        seen = np.ones(N, dtype=bool)
        if mask & MASK_KEY_PADDING and kv[b] == 0:
            seen[:] = False
        want = do[b][:, seen].sum(axis=1)
        assert np.max(np.abs(dV[b].sum(axis=1) - want)) <= 1e-11


@pytest.mark.parametrize("mask", MASKS)
def test_shift_invariances(mask):
    """K -> K + 1 u^T adds a per-row constant to the logits; V -> V + 1 c^T
    adds a per-row constant to dP.  Neither changes dS, so dQ and dK stay."""
    q, k, v, do = _rand(2, 2, 33, 6, seed=13)
    kv = np.array([20, 33], dtype=np.int32)
    g = np.random.default_rng(5)
    base = attention_bwd_ref(q, k, v, do, 0.4, mask, kv)
    u = g.standard_normal(6)
    c = g.standard_normal(6)
    ks = attention_bwd_ref(q, k + u, v, do, 0.4, mask, kv)
    vs = attention_bwd_ref(q, k, v + c, do, 0.4, mask, kv)
    for i in range(3):
        assert np.max(np.abs(ks[i] - base[i])) <= 1e-12
    for i in range(2):
        assert np.max(np.abs(vs[i] - base[i])) <= 1e-12
    assert np.array_equal(vs[2], base[2])


@pytest.mark.parametrize("mask", MASKS)
def test_dp_rowsum_is_do_dot_o(mask):
    q, k, v, do = _rand(2, 2, 40, 8, seed=14)
    kv = np.array([0, 25], dtype=np.int32)
    O, _ = attention_ref(q, k, v, 0.3, mask, kv)
    *_, D = attention_bwd_ref(q, k, v, do, 0.3, mask, kv)
    assert np.max(np.abs(D - (do * O).sum(axis=3))) <= 1e-12


def test_zero_upstream_gradient():
    q, k, v, _ = _rand(1, 2, 21, 4, seed=15)
    for t in attention_bwd_ref(q, k, v, np.zeros_like(q), 0.5, MASK_CAUSAL):
        assert np.all(t == 0.0)


def test_empty_rows_and_unseen_keys():
    """kv_len = 0: nothing is visible, every gradient is 0.  kv_len = 5: keys
    5.. get dK = dV = 0 and every row's dQ is finite."""
    q, k, v, do = _rand(2, 1, 12, 4, seed=16)
    kv = np.array([0, 5], dtype=np.int32)
    dQ, dK, dV, D = attention_bwd_ref(q, k, v, do, 0.5, MASK_KEY_PADDING | MASK_CAUSAL, kv)
    for t in (dQ[0], dK[0], dV[0], D[0]):
        assert np.all(t == 0.0)
    assert np.all(dK[1, :, 5:] == 0.0) and np.all(dV[1, :, 5:] == 0.0)
    assert np.all(np.isfinite(dQ))


# --- the block scan with recomputed probabilities ---------------------------------

@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("key_outer", [True, False])
def test_blocked_recomputation_any_partition_and_order(mask, key_outer):
    N, d = 70, 8
    q, k, v, do = _rand(1, 1, N, d, seed=17 + mask, qm=2.0)
    kvl = 45
    kv = np.array([kvl], dtype=np.int32)
    O, L = attention_ref(q, k, v, 0.35, mask, kv)
    want = attention_bwd_ref(q, k, v, do, 0.35, mask, kv)
    rng = np.random.default_rng(mask)
    for qb, kb in [(64, 64), (1, 7), (13, 3), (N, N), (32, 16)]:
        qbl = partition(N, qb)
        kbl = partition(N, kb)
        qbl = [qbl[i] for i in rng.permutation(len(qbl))]
        kbl = [kbl[i] for i in rng.permutation(len(kbl))]
        got = blocked_attention_bwd_ref(q[0, 0], k[0, 0], v[0, 0], O[0, 0], L[0, 0], do[0, 0],
                                        0.35, mask, kvl if mask & MASK_KEY_PADDING else None,
                                        qbl, kbl, key_outer)
        for i in range(4):
            assert np.max(np.abs(got[i] - want[i][0, 0])) <= 1e-12, (qb, kb, i)


def test_blocked_handles_empty_rows():
    q, k, v, do = _rand(1, 1, 10, 4, seed=18)
    O, L = attention_ref(q, k, v, 0.5, MASK_KEY_PADDING, np.array([0], dtype=np.int32))
    got = blocked_attention_bwd_ref(q[0, 0], k[0, 0], v[0, 0], O[0, 0], L[0, 0], do[0, 0],
                                    0.5, MASK_KEY_PADDING, 0)
    for t in got:
        assert np.all(t == 0.0)


def test_heads_subset_and_row_blocking_agree():
    q, k, v, do = _rand(2, 3, 45, 8, seed=19)
    full = attention_bwd_ref(q, k, v, do, 0.3, MASK_CAUSAL, row_block=512)
    part = attention_bwd_ref(q, k, v, do, 0.3, MASK_CAUSAL, heads=[(1, 2), (0, 0)], row_block=7)
    par = attention_bwd_ref(q, k, v, do, 0.3, MASK_CAUSAL, workers=3)
    for i in range(4):
        for b, h in [(1, 2), (0, 0)]:
            assert np.max(np.abs(part[i][b, h] - full[i][b, h])) <= 1e-12
        assert np.isnan(part[i][0, 1]).all()
        assert np.array_equal(par[i], full[i])


def test_row_subsets():
    """Only the listed rows contribute: dQ and D are exact on them, and under
    the causal mask the keys at or after the first row of a contiguous tail
    get their complete dK and dV."""
    N = 60
    q, k, v, do = _rand(1, 2, N, 8, seed=21)
    full = attention_bwd_ref(q, k, v, do, 0.3, MASK_CAUSAL)
    rows = np.array([3, 17, 40, 59])
    sub = attention_bwd_ref(q, k, v, do, 0.3, MASK_CAUSAL, rows=rows, row_block=3)
    assert np.max(np.abs(sub[0][:, :, rows] - full[0][:, :, rows])) <= 1e-13
    assert np.max(np.abs(sub[3][:, :, rows] - full[3][:, :, rows])) <= 1e-13
    others = np.setdiff1d(np.arange(N), rows)
    assert np.isnan(sub[0][:, :, others]).all() and np.isnan(sub[3][:, :, others]).all()
    tail = np.arange(44, N)
    sub = attention_bwd_ref(q, k, v, do, 0.3, MASK_CAUSAL, rows=tail)
    for i in (1, 2):
        assert np.max(np.abs(sub[i][:, :, 44:] - full[i][:, :, 44:])) <= 1e-13
        assert not np.allclose(sub[i][:, :, :44], full[i][:, :, :44])


@pytest.mark.parametrize("scale", [0.3, -0.3])
@pytest.mark.parametrize("mask", MASKS)
def test_magnitudes_bound_the_values(mask, scale):
    """Each magnitude is a sum of |terms|, so it is non-negative and bounds
    |value| (triangle inequality) for either sign of the scale, and equals
    it when every term is non-negative; asking for them changes no value."""
    q, k, v, do = _rand(2, 2, 41, 8, seed=22)
    kv = np.array([0, 30], dtype=np.int32)
    base = attention_bwd_ref(q, k, v, do, scale, mask, kv)
    *vals, mags = attention_bwd_ref(q, k, v, do, scale, mask, kv, magnitudes=True, row_block=9)
    for i, name in enumerate(("dq", "dk", "dv", "dps")):
        assert np.max(np.abs(vals[i] - base[i])) <= 1e-12
        finite = ~np.isnan(mags[name])
        assert np.all(mags[name][finite] >= 0.0), name
        assert np.all(mags[name] >= np.abs(vals[i]) * (1 - 1e-12) - 1e-300), name
    # dO >= 0 and V >= 0: every term of dV and of rowsum(dO * O) is >= 0.
    *vals, mags = attention_bwd_ref(q, k, np.abs(v), np.abs(do), scale, mask, kv,
                                    magnitudes=True)
    assert np.max(np.abs(mags["dv"] - vals[2])) <= 1e-12
    assert np.max(np.abs(mags["dps"] - vals[3])) <= 1e-12


def test_rejects_bad_arguments():
    q, k, v, do = _rand(1, 1, 4, 2, seed=20)
    with pytest.raises(ValueError):
        attention_bwd_ref(q, k, v, do, 1.0, 4)
    with pytest.raises(ValueError):
        attention_bwd_ref(q, k, v, do, 1.0, MASK_KEY_PADDING, None)
    with pytest.raises(ValueError):
        attention_bwd_ref(q, k, v, do[:, :, :3], 1.0)


# --- planted mistakes must be caught by the pins ---------------------------------

MUTATIONS = {
    "rowsum term dropped": ("ds = p * (dp - rs[:, None])", "ds = p * dp"),
    "rowsum of dP instead of dP * P": ("rs = (dp * p).sum(axis=1)", "rs = dp.sum(axis=1)"),
    "dS sign flipped": ("ds = p * (dp - rs[:, None])", "ds = p * (rs[:, None] - dp)"),
    "dQ without scale": ("dq[rr] = (ds @ kh[:kmax]) * scale", "dq[rr] = (ds @ kh[:kmax])"),
    "dK without scale": ("dk[:kmax] += (ds.T @ qh[rr]) * scale", "dk[:kmax] += (ds.T @ qh[rr])"),
    "dK from K instead of Q": ("dk[:kmax] += (ds.T @ qh[rr]) * scale",
                               "dk[:kmax] += (ds.T @ kh[rr]) * scale"),
    "dV from V instead of dO": ("dv[:kmax] += p.T @ doh[rr]", "dv[:kmax] += p.T @ vh[rr]"),
    "dP from K instead of V": ("dp = doh[rr] @ vh[:kmax].T", "dp = doh[rr] @ kh[:kmax].T"),
    "P not normalised": ("p[ok] = e / e.sum(axis=1, keepdims=True)", "p[ok] = e"),
    "mask dropped in the backward": ("s = np.where(_visible(rr, cols, causal, n_vis), s, -np.inf)",
                                     "s = s"),
    "causal mask off by one": ("cols[None, :] <= rows[:, None]", "cols[None, :] < rows[:, None]"),
    "scale missing from the logits": ("s = (qh[rr] @ kh[:kmax].T) * scale",
                                      "s = (qh[rr] @ kh[:kmax].T)"),
    "dV with unscaled rows of P^T": ("dv[:kmax] += p.T @ doh[rr]",
                                     "dv[:kmax] += p.T @ doh[rr] * 0.5"),
}


def _bwd_pins_pass(ref) -> bool:
    """Finite differences (all masks, empty rows) and the Q = 0 closed form."""
    try:
        for mask in MASKS:
            q, k, v, do = _rand(2, 1, 5, 3, seed=60 + mask)
            kv = np.array([0, 4], dtype=np.int32)
            got = ref(q, k, v, do, 0.8, mask, kv)
            for g, w in zip(got[:3], _fd_grads(q, k, v, do, 0.8, mask, kv)):
                if not np.max(np.abs(g - w)) <= 2e-7:
                    return False
        return True
    except Exception:
        return False


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name):
    import inspect
    src = inspect.getsource(bwd_mod)
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    src = src.replace("from .attention_ref import", "from oracle.attention_ref import")
    ns = {"__name__": "mutated_bwd_oracle"}
    exec(compile(src.replace(old, new), "<mutated bwd oracle>", "exec"), ns)
    assert _bwd_pins_pass(bwd_mod.attention_bwd_ref), "pins must pass on the unmodified oracle"
    assert not _bwd_pins_pass(ns["attention_bwd_ref"]), f"planted mistake not caught: {name}"
