"""GPU parity of the backward pass: the HIP gradients against the CPU oracle.

Every test runs the forward and then the backward through the C ABI and
compares dQ, dK, dV (and the row sums D) element by element with the fp64
oracle of the gradient equations; the long-context workload is compared in
full on one head plus closed forms and invariants that hold at any size.
Gradient buffers are pre-filled with NaN so an unwritten element fails.
"""
import numpy as np
import pytest

from fa_inputs import (MASK_CAUSAL, MASK_KEY_PADDING, MASK_NONE, WORKLOADS, make_bwd_inputs,
                       make_grad_out, make_raw, to_f64)
from gpu_util import compare_grads, run_bwd_gpu, say, to_dev
from oracle import attention_bwd_ref

pytestmark = pytest.mark.gpu

MASKS = [MASK_NONE, MASK_CAUSAL, MASK_KEY_PADDING, MASK_CAUSAL | MASK_KEY_PADDING]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")
    import exact_attention_92_amd as fa
    fa.load_library()


def _oracle(x, scale, mask, rows=None, workers=16):
    """fp64 gradients and their magnitudes: (values, magnitudes) dicts."""
    dq, dk, dv, dps, mag = attention_bwd_ref(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]),
                                             to_f64(x["do"]), scale, mask, x.get("kv_lens"),
                                             rows=rows, workers=workers, magnitudes=True)
    return {"dq": dq, "dk": dk, "dv": dv, "dps": dps}, mag


def _raw_bwd(B, H, N, d, seed, **kw):
    x = make_raw(B, H, N, d, "bf16", seed, **kw)
    x["do"] = make_grad_out(B, H, N, d, "bf16", seed)
    return x


@pytest.mark.parametrize("name", [n for n in WORKLOADS
                                  if WORKLOADS[n].dtype == "bf16" and "n65536" not in n])
def test_workload_full_parity(name):
    wl = WORKLOADS[name]
    say(f"[bwd parity] {name}")
    x = make_bwd_inputs(wl)
    g = run_bwd_gpu(x, wl.scale, wl.mask_kind)
    ref, mag = _oracle(x, wl.scale, wl.mask_kind)
    compare_grads(g, ref, mag, name, keys=("dq", "dk", "dv", "dps"), bulk=True)


def test_long_context_tail_keys_sampled_rows_and_invariants():
    """N = 65536 causal: the last 2048 keys are seen only by the last 2048
    rows, so the oracle over those rows gives their complete dK and dV;
    dQ is compared on sampled rows; the key and value gradient sums are
    checked on every head."""
    wl = WORKLOADS["bf16_b1h8_n65536_d128_causal"]
    say(f"[bwd parity] {wl.name}: tail keys, sampled rows, invariants")
    x = make_bwd_inputs(wl)
    g = run_bwd_gpu(x, wl.scale, wl.mask_kind)
    for name in ("dq", "dk", "dv"):
        assert not np.isnan(g[name]).any(), name
    # Every row sees key 0, so the rows of dS sum to zero and the rows of P
    # sum to one: sum_c dK_c = 0 and sum_c dV_c = sum_r dO_r, per head.
    do = to_f64(x["do"])
    assert np.max(np.abs(g["dv"].sum(axis=2) - do.sum(axis=2))) <= 2e-2 * np.sqrt(wl.N), "sum dV"
    dk_abs = np.abs(g["dk"]).sum(axis=2)
    assert np.all(np.abs(g["dk"].sum(axis=2)) <= 1e-2 * dk_abs), "sum dK"
    T = 2048
    ref, mag = _oracle(x, wl.scale, wl.mask_kind, rows=np.arange(wl.N - T, wl.N))
    tail = lambda t: {n: t[n][:, :, -T:] for n in ("dq", "dk", "dv", "dps")}
    compare_grads(tail(g), tail(ref), tail(mag), wl.name + " tail",
                  keys=("dq", "dk", "dv", "dps"), bulk=True)
    rows = np.unique(np.r_[0:130, np.random.default_rng(2).integers(0, wl.N, 200)])
    ref, mag = _oracle(x, wl.scale, wl.mask_kind, rows=rows)
    pick = lambda t: {n: t[n][:, :, rows] for n in ("dq", "dps")}
    compare_grads(pick(g), pick(ref), pick(mag), wl.name + " sampled rows", keys=("dq", "dps"))


@pytest.mark.parametrize("d", [64, 128])
def test_q_zero_closed_form_long_causal(d):
    """Q = 0: P_r is uniform over keys 0..r.  Then dK = 0 exactly,
    dV_c = sum_{r >= c} dO_r / (r + 1), and
    dQ_r = scale / (r + 1) * sum_{c <= r} (dO_r . (v_c - mean_{c' <= r} v)) k_c.
    The magnitudes for the error bound are the same sums over |terms|."""
    B, H, N = 1, 2, 65536
    say(f"[bwd closed form] Q=0 causal N={N} d={d}")
    x = _raw_bwd(B, H, N, d, seed=41)
    x["q"] = np.zeros_like(x["q"])
    scale = d ** -0.5
    g = run_bwd_gpu(x, scale, MASK_CAUSAL)
    assert np.all(g["dk"] == 0.0)
    do, v, k = to_f64(x["do"]), to_f64(x["v"]), to_f64(x["k"])
    cnt = np.arange(1, N + 1, dtype=np.float64)
    w = do / cnt[None, None, :, None]
    suffix = lambda t: np.flip(np.cumsum(np.flip(t, axis=2), axis=2), axis=2)
    dv_ref = suffix(w)
    dv_mag = suffix(np.abs(w))
    compare_grads({"dv": g["dv"]}, {"dv": dv_ref}, {"dv": dv_mag}, f"Q=0 dV d={d}",
                  keys=("dv",), bulk=True)
    rows = np.unique(np.r_[0:40, np.random.default_rng(1).integers(0, N, 60), N - 40:N])
    dq_ref = np.zeros((B, H, len(rows), d))
    dq_mag = np.zeros((B, H, len(rows), d))
    for h in range(H):
        for i, r in enumerate(rows):
            vv, kk, dr = v[0, h, :r + 1], k[0, h, :r + 1], do[0, h, r]
            ds = (vv - vv.mean(axis=0)) @ dr / (r + 1)       # dS_rc = P (dP - D)
            dq_ref[0, h, i] = scale * (ds @ kk)
            a_d = np.abs(dr) @ np.abs(vv).mean(axis=0)       # sum_t |dO| (P |V|)
            dq_mag[0, h, i] = scale * (np.abs(ds) @ np.abs(kk) + a_d * np.abs(kk).mean(axis=0))
    compare_grads({"dq": g["dq"][:, :, rows]}, {"dq": dq_ref}, {"dq": dq_mag}, f"Q=0 dQ d={d}",
                  keys=("dq",))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 4, 63, 65, 127, 129, 1000])
def test_ragged_lengths_all_masks(d, N):
    B, H = 2, 3
    x = _raw_bwd(B, H, N, d, seed=2000 + N + d, q_mult=2.0,
                 kv_len_range=(max(0, N // 2 - 3), N))
    for mask in MASKS:
        what = f"N={N} d={d} mask={mask} kv={x['kv_lens'].tolist()}"
        g = run_bwd_gpu(x, d ** -0.5, mask)
        ref, mag = _oracle(x, d ** -0.5, mask)
        compare_grads(g, ref, mag, what, keys=("dq", "dk", "dv", "dps"))


def test_kv_len_edges_and_clamping():
    N, d = 300, 128
    lens = [0, 1, 63, 64, 65, 127, 128, 129, N]
    x = _raw_bwd(len(lens), 2, N, d, seed=78)
    x["kv_lens"] = np.array(lens, dtype=np.int32)
    for mask in (MASK_KEY_PADDING, MASK_KEY_PADDING | MASK_CAUSAL):
        g = run_bwd_gpu(x, d ** -0.5, mask)
        ref, mag = _oracle(x, d ** -0.5, mask)
        compare_grads(g, ref, mag, f"kv_len edges mask={mask}")
        # Batch entry 0 sees no key at all: every gradient is exactly 0.
        for name in ("dq", "dk", "dv"):
            assert np.all(g[name][0] == 0.0), name
        for b, kl in enumerate(lens):
            assert np.all(g["dk"][b, :, kl:] == 0.0) and np.all(g["dv"][b, :, kl:] == 0.0)
    x["kv_lens"] = np.array([-5, N + 100] + lens[2:], dtype=np.int32)
    g = run_bwd_gpu(x, d ** -0.5, MASK_KEY_PADDING)
    x2 = dict(x, kv_lens=np.clip(x["kv_lens"], 0, N).astype(np.int32))
    compare_grads(g, *_oracle(x2, d ** -0.5, MASK_KEY_PADDING), "kv_len clamped")


def test_hidden_keys_may_hold_non_finite_values():
    N, d = 200, 64
    x = _raw_bwd(2, 2, N, d, seed=6)
    x["kv_lens"] = np.array([70, 131], dtype=np.int32)
    y = dict(x)
    y["k"], y["v"] = x["k"].copy(), x["v"].copy()
    for b, kl in enumerate(x["kv_lens"]):
        y["k"][b, :, kl:] = 0x7FC0   # NaN
        y["v"][b, :, kl:] = 0x7F80   # +inf
    for mask in (MASK_KEY_PADDING, MASK_KEY_PADDING | MASK_CAUSAL):
        ga = run_bwd_gpu(x, 0.125, mask)
        gb = run_bwd_gpu(y, 0.125, mask)
        for name in ("dq", "dk", "dv", "dps"):
            assert np.array_equal(ga[name], gb[name]), (mask, name)


@pytest.mark.parametrize("scale", [-0.3, 0.0, 1e-35, 2.0])
def test_unusual_scales(scale):
    x = _raw_bwd(1, 2, 190, 64, seed=10)
    for mask in (MASK_NONE, MASK_CAUSAL):
        g = run_bwd_gpu(x, scale, mask)
        ref, mag = _oracle(x, scale, mask)
        compare_grads(g, ref, mag, f"scale={scale} mask={mask}",
                      keys=("dv",) if abs(scale) < 1e-30 else ("dq", "dk", "dv"))
        if abs(scale) < 1e-30:
            # The exact dQ and dK are 0 * (...); the kernel's are below 1e-28.
            assert np.max(np.abs(g["dq"])) < 1e-28 and np.max(np.abs(g["dk"])) < 1e-28


def test_bitwise_deterministic():
    wl = WORKLOADS["bf16_b4h16_n1024_d64_causal"]
    x = make_bwd_inputs(wl)
    runs = [run_bwd_gpu(x, wl.scale, wl.mask_kind) for _ in range(3)]
    for r in runs[1:]:
        for name in ("dq", "dk", "dv", "dps"):
            assert np.array_equal(r[name], runs[0][name]), name


def test_non_default_stream():
    import torch

    import exact_attention_92_amd as fa
    x = _raw_bwd(2, 4, 777, 128, seed=22)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = fa.attention(q, k, v, 128 ** -0.5, fa.FA_MASK_CAUSAL)
        dq, dk, dv = fa.attention_grad(q, k, v, o, lse, do, 128 ** -0.5, fa.FA_MASK_CAUSAL)
    s.synchronize()
    from gpu_util import o_to_f64
    g = {"dq": o_to_f64(dq), "dk": o_to_f64(dk), "dv": o_to_f64(dv)}
    compare_grads(g, *_oracle(x, 128 ** -0.5, MASK_CAUSAL), "side stream")


def test_errors_write_nothing():
    import torch

    import exact_attention_92_amd as fa
    q = torch.zeros((1, 1, 64, 96), dtype=torch.bfloat16, device="cuda")
    outs = [torch.full_like(q, float("nan")) for _ in range(3)]
    dps = torch.full((1, 1, 64), float("nan"), device="cuda")
    lse = torch.zeros((1, 1, 64), device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fa_bwd(q, q, q, q, lse, q, *outs, dps, 0.1)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    with pytest.raises(fa.FaError) as e:
        fa.fa_bwd(q, q, q, q, lse, q, *outs, dps, float("nan"))
    assert e.value.status == fa.FA_ERR_INVALID_ARG
    torch.cuda.synchronize()
    for t in outs + [dps]:
        assert torch.isnan(t).all()


BWD_EDGES = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 383, 511, 513]


@pytest.mark.parametrize("chunk", range(3))
def test_random_shapes_masks_and_scales(chunk):
    """Seeded random cases: each draws d, B, H, N (half of them at the 32-,
    64-, 128- and 256-row block edges), the mask, the key lengths (down to 0)
    and the scale from its own seed; dQ, dK, dV and the row sums element by
    element against the oracle."""
    for seed in range(900 + 10 * chunk, 900 + 10 * chunk + 10):
        rng = np.random.default_rng(seed)
        d = int(rng.choice([64, 128]))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        N = int(rng.choice(BWD_EDGES)) if rng.random() < 0.5 else int(rng.integers(1, 800))
        mask = int(rng.integers(0, 4))
        scale = float(d ** -0.5 * rng.choice([1.0, 1.0, -0.7, 2.5]))
        kv_range = (0, N) if mask & MASK_KEY_PADDING else None
        x = _raw_bwd(B, H, N, d, seed, q_mult=2.0, kv_len_range=kv_range)
        kv = None if x["kv_lens"] is None else x["kv_lens"].tolist()
        what = f"seed={seed} B={B} H={H} N={N} d={d} mask={mask} kv={kv} scale={scale:.4f}"
        say(what)
        g = run_bwd_gpu(x, scale, mask)
        ref, mag = _oracle(x, scale, mask)
        compare_grads(g, ref, mag, what, keys=("dq", "dk", "dv", "dps"))
