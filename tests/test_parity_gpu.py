"""GPU parity: the HIP path against the CPU oracle on the same seeded bytes.

Every test here runs the kernels through the C ABI (ctypes binding) and
compares element by element with the fp64 oracle; the N = 65536 workload is
compared on every element, on sampled rows, and against a closed form that
holds at any size.  Output
buffers are pre-filled with NaN so an unwritten element fails.
"""
import json
import math
import os

import numpy as np
import pytest

from fa_inputs import (MASK_CAUSAL, MASK_KEY_PADDING, MASK_NONE, WORKLOADS, f32_to_bf16_bits,
                       make_inputs, make_raw, to_f64)
from gpu_util import compare, o_to_f64, run_gpu, say, to_dev
from oracle import attention_ref

pytestmark = pytest.mark.gpu

MASKS = [MASK_NONE, MASK_CAUSAL, MASK_KEY_PADDING, MASK_CAUSAL | MASK_KEY_PADDING]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")
    import exact_attention_92_amd as fa
    fa.load_library()
    say(f"device: {torch.cuda.get_device_name(0)}")


def _oracle(x, scale, mask, rows=None, heads=None):
    return attention_ref(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]), scale, mask,
                         x.get("kv_lens"), rows=rows, heads=heads, workers=16)


@pytest.mark.parametrize("name", [n for n in WORKLOADS if "n65536" not in n])
def test_workload_full_parity(name):
    wl = WORKLOADS[name]
    say(f"[parity] {name}")
    x = make_inputs(wl)
    O, L = run_gpu(x, wl.scale, wl.mask_kind)
    Or, Lr = _oracle(x, wl.scale, wl.mask_kind)
    compare(O, L, Or, Lr, wl.dtype, name)


def test_long_context_sampled_rows():
    wl = WORKLOADS["bf16_b1h8_n65536_d128_causal"]
    say(f"[parity] {wl.name} (sampled rows)")
    x = make_inputs(wl)
    O, L = run_gpu(x, wl.scale, wl.mask_kind)
    g = np.random.default_rng(0)
    rows = np.unique(np.r_[0:130, g.integers(0, wl.N, 300), wl.N - 130:wl.N])
    Or, Lr = _oracle(x, wl.scale, wl.mask_kind, rows=rows)
    compare(O[:, :, rows], L[:, :, rows], Or, Lr, wl.dtype, wl.name + " sampled")


def test_long_context_full_tensor():
    """Every element of the N = 65536 workload (8 heads x 65536 rows) against
    the oracle; the host computes the oracle's rows in chunks of 4096 per
    head, in parallel (each chunk is the oracle's own arithmetic)."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    wl = WORKLOADS["bf16_b1h8_n65536_d128_causal"]
    say(f"[parity] {wl.name} (full tensor)")
    x = make_inputs(wl)
    O, L = run_gpu(x, wl.scale, wl.mask_kind)
    q, k, v = (to_f64(x[n]) for n in "qkv")
    Or, Lr = np.full_like(O, np.nan), np.full_like(L, np.nan)
    step = 4096

    def chunk(unit):
        b, h, r0 = unit
        rows = np.arange(r0, min(wl.N, r0 + step))
        o, lse = attention_ref(q, k, v, wl.scale, wl.mask_kind, x.get("kv_lens"), rows=rows,
                               heads=[(b, h)])
        Or[b, h, rows], Lr[b, h, rows] = o[b, h], lse[b, h]

    units = [(b, h, r0) for b in range(wl.B) for h in range(wl.H)
             for r0 in range(wl.N - step, -1, -step)]      # longest rows first
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        list(ex.map(chunk, units))
    compare(O, L, Or, Lr, wl.dtype, wl.name + " full tensor")


@pytest.mark.parametrize("d", [64, 128])
def test_q_zero_closed_form_long_causal(d):
    """Q = 0: P is uniform over the visible prefix, so O_r is the mean of
    V[0..r] and LSE_r = ln(r + 1), at full length N = 65536."""
    B, H, N = 1, 2, 65536
    say(f"[closed form] Q=0 causal N={N} d={d}")
    x = make_raw(B, H, N, d, "bf16", seed=31)
    x["q"] = np.zeros_like(x["q"])
    O, L = run_gpu(x, d ** -0.5, MASK_CAUSAL)
    v = to_f64(x["v"])
    cnt = np.arange(1, N + 1, dtype=np.float64)
    Or = np.cumsum(v, axis=2) / cnt[None, None, :, None]
    Lr = np.broadcast_to(np.log(cnt), (B, H, N))
    compare(O, L, Or, Lr, "bf16", "Q=0 causal prefix mean")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_worked_example(dtype):
    """Logits [1, 2, 3, 0] of the page's worked example as query 0's scores
    (scale 1/8, q0 = 8 e_0, K[:, 0] = [1, 2, 3, 0]); V = identity in the
    first four dims, so O_0[:4] is the softmax and LSE_0 = 3 + ln l2."""
    path = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")
    ex = json.load(open(path))
    N, d = 4, 64
    q = np.zeros((1, 1, N, d), np.float32)
    k = np.zeros((1, 1, N, d), np.float32)
    v = np.zeros((1, 1, N, d), np.float32)
    q[0, 0, 0, 0] = 8.0
    k[0, 0, :, 0] = ex["logits"]
    v[0, 0, :, :N] = np.eye(N)
    x = {"q": q, "k": k, "v": v, "kv_lens": None}
    if dtype == "bf16":
        x = {n: f32_to_bf16_bits(x[n]) for n in "qkv"}
    O, L = run_gpu(x, 0.125, MASK_NONE)
    l2 = math.fsum(math.exp(e) for e in ex["after_block_2"]["l_exponents"])
    want = np.exp(np.array(ex["logits"], dtype=np.float64) - 3.0) / l2
    tol = 1e-2 if dtype == "bf16" else 1e-6
    assert np.max(np.abs(O[0, 0, 0, :N] - want)) <= tol
    assert abs(L[0, 0, 0] - (3.0 + math.log(l2))) <= (1e-3 if dtype == "bf16" else 1e-6)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 4, 63, 65, 127, 129, 1000])
def test_ragged_lengths_all_masks(dtype, d, N):
    B, H = 2, 3
    x = make_raw(B, H, N, d, dtype, seed=1000 + N + d, q_mult=2.0,
                 kv_len_range=(max(0, N // 2 - 3), N))
    for mask in MASKS:
        what = f"{dtype} N={N} d={d} mask={mask} kv={x['kv_lens'].tolist()}"
        O, L = run_gpu(x, d ** -0.5, mask)
        Or, Lr = _oracle(x, d ** -0.5, mask)
        compare(O, L, Or, Lr, dtype, what)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kv_len_edges(dtype):
    N, d = 300, 128
    lens = [0, 1, 63, 64, 65, 127, 128, 129, N]
    x = make_raw(len(lens), 2, N, d, dtype, seed=77)
    x["kv_lens"] = np.array(lens, dtype=np.int32)
    for mask in (MASK_KEY_PADDING, MASK_KEY_PADDING | MASK_CAUSAL):
        O, L = run_gpu(x, d ** -0.5, mask)
        Or, Lr = _oracle(x, d ** -0.5, mask)
        compare(O, L, Or, Lr, dtype, f"{dtype} kv_len edges mask={mask}")
    # Out-of-range lengths are clamped to [0, N].
    x["kv_lens"] = np.array([-5, N + 100] + lens[2:], dtype=np.int32)
    O, L = run_gpu(x, d ** -0.5, MASK_KEY_PADDING)
    x2 = dict(x, kv_lens=np.clip(x["kv_lens"], 0, N).astype(np.int32))
    Or, Lr = _oracle(x2, d ** -0.5, MASK_KEY_PADDING)
    compare(O, L, Or, Lr, dtype, f"{dtype} kv_len clamped")


def test_hidden_keys_may_hold_non_finite_values():
    """Keys at or past kv_len never influence the output, whatever they hold."""
    N, d = 200, 64
    x = make_raw(2, 2, N, d, "bf16", seed=5)
    x["kv_lens"] = np.array([70, 131], dtype=np.int32)
    y = {n: x[n].copy() for n in "qkv"}
    y["kv_lens"] = x["kv_lens"]
    for b, kl in enumerate(x["kv_lens"]):
        y["k"][b, :, kl:] = 0x7FC0   # NaN
        y["v"][b, :, kl:] = 0x7F80   # +inf
    Oa, La = run_gpu(x, 0.125, MASK_KEY_PADDING)
    Ob, Lb = run_gpu(y, 0.125, MASK_KEY_PADDING)
    assert np.array_equal(Oa, Ob) and np.array_equal(La, Lb)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [-0.3, 0.0, 1e-35, 2.0])
def test_unusual_scales(dtype, scale):
    x = make_raw(1, 2, 190, 64, dtype, seed=9)
    for mask in (MASK_NONE, MASK_CAUSAL):
        O, L = run_gpu(x, scale, mask)
        Or, Lr = _oracle(x, scale, mask)
        compare(O, L, Or, Lr, dtype, f"{dtype} scale={scale} mask={mask}")


def test_bitwise_deterministic():
    wl = WORKLOADS["bf16_b4h16_n1024_d64_causal"]
    x = make_inputs(wl)
    outs = [run_gpu(x, wl.scale, wl.mask_kind) for _ in range(3)]
    for O, L in outs[1:]:
        assert np.array_equal(O, outs[0][0]) and np.array_equal(L, outs[0][1])


def test_non_default_stream_and_async():
    import torch

    import exact_attention_92_amd as fa
    x = make_raw(2, 4, 777, 128, "bf16", seed=21)
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = fa.attention(q, k, v, 128 ** -0.5, fa.FA_MASK_CAUSAL)
    s.synchronize()
    Or, Lr = _oracle(x, 128 ** -0.5, MASK_CAUSAL)
    compare(o_to_f64(o), lse.cpu().numpy().astype(np.float64), Or, Lr, "bf16", "side stream")


def test_errors_write_nothing():
    import torch

    import exact_attention_92_amd as fa
    q = torch.zeros((1, 1, 64, 80), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, 1, 64), float("nan"), device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd(q, q, q, o, lse, 0.1)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    q = torch.zeros((2, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, float("nan"))
    lse = torch.full((2, 1, 64), float("nan"), device="cuda")
    lib = fa.load_library()
    import ctypes
    st = lib.fa_fwd(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(q.data_ptr()),
                    ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(o.data_ptr()),
                    ctypes.c_void_p(lse.data_ptr()), 2, 1, 64, 64, ctypes.c_float(0.1),
                    fa.FA_MASK_KEY_PADDING, None, None)
    assert st == fa.FA_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.isnan(o).all() and torch.isnan(lse).all()
