"""GPU parity of the general bf16 forward (fa_fwd_general): N_q != N_k with
the queries at the last N_q key positions, sliding windows and strided
layouts, against the general-mask oracle.

Bars, per element of O: 2^-8 |O_ref| (O's own bf16 rounding) + 2^-7 (P|V|)
(the probabilities are rounded to bf16, relative 2^-8 each, and normalised by
the sum of the rounded values, another 2^-8) + 1e-5 (P|V|) (fp32 sums); LSE
within 1e-3; empty rows exactly O = 0 and LSE = -inf; relative Frobenius
<= 5e-3 as for the named bf16 workloads.  (The flat 1e-2 max-abs of the named
workloads is not a bound when a short window leaves one V row dominant with
|O| in [2, 4): its bf16 rounding alone can reach 7.8e-3.)  Outputs are
pre-filled with NaN so an unwritten element fails."""
import numpy as np
import pytest

from fa_inputs import MASK_CAUSAL, MASK_KEY_PADDING, MASK_NONE, make_raw, to_f64
from gpu_util import compare_bound as compare
from gpu_util import o_to_f64, say, to_dev
from oracle import attention_general_ref

pytestmark = pytest.mark.gpu

MASKS = [MASK_NONE, MASK_CAUSAL, MASK_KEY_PADDING, MASK_CAUSAL | MASK_KEY_PADDING]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")
    import exact_attention_92_amd as fa
    fa.load_library()


def _inputs(B, H, Nq, Nk, d, seed, kv_range=None):
    xq = make_raw(B, H, Nq, d, "bf16", seed=seed, q_mult=2.0)
    xk = make_raw(B, H, Nk, d, "bf16", seed=seed + 1, kv_len_range=kv_range)
    return {"q": xq["q"], "k": xk["k"], "v": xk["v"], "kv_lens": xk["kv_lens"]}


def run_general(x, scale, mask, window, layout="bhnd"):
    import torch

    import exact_attention_92_amd as fa

    def dev(a):
        t = to_dev(a)
        if layout == "bnhd":        # same values, stored [B, N, H, d]
            t = t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        return t
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    B, H, Nq, d = q.shape
    o = torch.full((B, Nq, H, d) if layout == "bnhd" else (B, H, Nq, d), float("nan"),
                   dtype=torch.bfloat16, device="cuda")
    if layout == "bnhd":
        o = o.permute(0, 2, 1, 3)
    lse = torch.full((B, H, Nq), float("nan"), device="cuda")
    kv = None if x.get("kv_lens") is None else torch.from_numpy(x["kv_lens"]).cuda()
    fa.fa_fwd_general(q, k, v, o, lse, scale, mask, window, kv)
    torch.cuda.synchronize()
    return o_to_f64(o.contiguous()), lse.cpu().numpy().astype(np.float64)


def oracle(x, scale, mask, window):
    return attention_general_ref(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]), scale, mask,
                                 window, x.get("kv_lens"), magnitudes=True)


@pytest.mark.parametrize("d", [64, 128])
def test_degenerate_case_is_fa_fwd_bitwise(d):
    import torch

    import exact_attention_92_amd as fa
    x = make_raw(2, 3, 517, d, "bf16", seed=70, kv_len_range=(200, 517))
    for mask in MASKS:
        Og, Lg = run_general(x, d ** -0.5, mask, -1)
        q, k, v = (to_dev(x[n]) for n in "qkv")
        o = torch.empty_like(q)
        lse = torch.empty((2, 3, 517), device="cuda")
        fa.fa_fwd(q, k, v, o, lse, d ** -0.5, mask, torch.from_numpy(x["kv_lens"]).cuda())
        torch.cuda.synchronize()
        assert np.array_equal(Og, o_to_f64(o)) and np.array_equal(Lg, lse.cpu().numpy())


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nq,Nk", [(1, 300), (65, 1000), (200, 129), (300, 77), (256, 256)])
def test_lengths_masks_windows(d, Nq, Nk):
    x = _inputs(2, 2, Nq, Nk, d, seed=71 + Nq + Nk + d, kv_range=(max(1, Nk // 3), Nk))
    for mask in MASKS:
        for window in (-1, 0, 17, 200):
            O, L = run_general(x, d ** -0.5, mask, window)
            compare(O, L, oracle(x, d ** -0.5, mask, window),
                    f"Nq={Nq} Nk={Nk} d={d} mask={mask} W={window}")


def test_strided_bnhd_layout_is_bitwise_the_contiguous_result():
    x = _inputs(2, 4, 333, 333, 128, seed=90)
    for mask, window in ((MASK_CAUSAL, -1), (MASK_CAUSAL, 64), (MASK_NONE, 10)):
        Oa, La = run_general(x, 128 ** -0.5, mask, window, "bhnd")
        Ob, Lb = run_general(x, 128 ** -0.5, mask, window, "bnhd")
        assert np.array_equal(Oa, Ob) and np.array_equal(La, Lb)
        compare(Ob, Lb, oracle(x, 128 ** -0.5, mask, window), f"BNHD mask={mask} W={window}")


def test_long_sliding_window():
    x = _inputs(1, 1, 8192, 8192, 128, seed=91)
    say("[general] N=8192 causal window 1024")
    O, L = run_general(x, 128 ** -0.5, MASK_CAUSAL, 1024)
    compare(O, L, oracle(x, 128 ** -0.5, MASK_CAUSAL, 1024), "N=8192 causal W=1024")


def _sample_rows(N, W):
    rows = {0, 1, 31, 32, 127, 128, W - 1, W, W + 1, N - 2, N - 1}
    rows.update(np.linspace(0, N - 1, 48).astype(int).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < N))


@pytest.mark.parametrize("name", ["bf16_b1h8_n65536_d128_causal_w4096",
                                  "bf16_b2h32_n4096_d128_causal_bnhd"])
def test_general_bench_workload_sampled_rows(name):
    """The general workloads at full size, in the layout and launch the bench
    times, on a sample of query rows of every head."""
    from fa_inputs import GENERAL_WORKLOADS, make_inputs
    wl = GENERAL_WORKLOADS[name]
    say(f"[general] {name}")
    x = make_inputs(wl)
    O, L = run_general(x, wl.scale, wl.mask_kind, wl.window_left, wl.layout)
    rows = _sample_rows(wl.N, max(wl.window_left, 64))
    ref = attention_general_ref(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]), wl.scale,
                                wl.mask_kind, wl.window_left, x["kv_lens"], magnitudes=True,
                                rows=rows)
    compare(O[:, :, rows], L[:, :, rows], ref, f"{name} ({len(rows)} rows per head)")
