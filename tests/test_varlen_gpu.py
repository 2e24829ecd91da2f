"""GPU parity of the packed variable-length forward (fa_fwd_varlen) and of
the head dimensions 32, 96 and 256 (fa_fwd, fa_fwd_general), against the
oracle, with the element bound of the general forward (O's bf16 rounding
plus P rounded to bf16, see gpu_util.compare_bound).  Outputs are
pre-filled with NaN so an unwritten element fails."""
import numpy as np
import pytest

from fa_inputs import MASK_CAUSAL, MASK_KEY_PADDING, MASK_NONE, make_packed, make_raw, to_f64
from gpu_util import compare_bound, o_to_f64, say, to_dev
from oracle import attention_general_ref, attention_varlen_ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")
    import exact_attention_92_amd as fa
    fa.load_library()


def run_varlen(x, max_q, scale, mask, window):
    import torch

    import exact_attention_92_amd as fa
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    total_q, H, d = q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((H, total_q), float("nan"), device="cuda")
    cu_q = torch.from_numpy(x["cu_q"]).cuda()
    cu_k = torch.from_numpy(x["cu_k"]).cuda()
    fa.fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, max_q, scale, mask, window)
    torch.cuda.synchronize()
    return o_to_f64(o), lse.cpu().numpy().astype(np.float64)


def check_varlen(x, scale, mask, window, what, max_q=None):
    lens = np.diff(x["cu_q"])
    max_q = int(lens.max()) if max_q is None else max_q
    O, L = run_varlen(x, max_q, scale, mask, window)
    Or, Lr, M = attention_varlen_ref(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]),
                                     x["cu_q"], x["cu_k"], scale, mask, window, magnitudes=True)
    # Rows as [H, total_q, d] to match LSE's [H, total_q].
    t = (1, 0, 2)
    compare_bound(O.transpose(t), L, (Or.transpose(t), Lr, M.transpose(t)), what)


LENS = ([0, 1, 63, 64, 65, 200, 257, 10, 300],      # queries per sequence
        [5, 1, 63, 100, 65, 129, 257, 0, 1000])    # keys per sequence (10 queries, no keys)


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
def test_ragged_packing(d):
    x = make_packed(*LENS, H=3, d=d, seed=200 + d, q_mult=2.0)
    for mask in (MASK_NONE, MASK_CAUSAL):
        for window in (-1, 0, 37):
            check_varlen(x, d ** -0.5, mask, window, f"ragged d={d} mask={mask} W={window}")


def test_large_batch_uses_the_wide_workgroups():
    # 32 sequences of 1000-2000 rows, 8 heads: the 8-wave launch.
    g = np.random.default_rng(7)
    lq = g.integers(1000, 2000, size=32, endpoint=True)
    lk = lq + g.integers(0, 64, size=32)
    x = make_packed(lq, lk, H=8, d=128, seed=210)
    say(f"[varlen] 32 sequences, total_q={int(lq.sum())}")
    check_varlen(x, 128 ** -0.5, MASK_CAUSAL, -1, "32 seqs causal")


def test_equal_lengths_match_the_general_forward_bitwise():
    import torch

    import exact_attention_92_amd as fa
    B, H, n, d = 3, 4, 333, 128
    x = make_packed([n] * B, [n] * B, H=H, d=d, seed=220)
    for mask, window in ((MASK_CAUSAL, -1), (MASK_NONE, 50)):
        O, L = run_varlen(x, n, d ** -0.5, mask, window)
        # The same bytes viewed as [B, H, n, d] through strides.
        q, k, v = (to_dev(x[t]).view(B, n, H, d).permute(0, 2, 1, 3) for t in "qkv")
        o = torch.full((B, n, H, d), float("nan"), dtype=torch.bfloat16,
                       device="cuda").permute(0, 2, 1, 3)
        lse = torch.full((B, H, n), float("nan"), device="cuda")
        fa.fa_fwd_general(q, k, v, o, lse, d ** -0.5, mask, window)
        torch.cuda.synchronize()
        Og = o_to_f64(o.permute(0, 2, 1, 3).contiguous()).reshape(B * n, H, d)
        Lg = lse.cpu().numpy().transpose(1, 0, 2).reshape(H, B * n)
        assert np.array_equal(O, Og) and np.array_equal(L, Lg)


def test_rows_past_max_seqlen_are_not_written():
    x = make_packed([100, 300], [100, 300], H=2, d=64, seed=230)
    O, L = run_varlen(x, 256, 0.125, MASK_CAUSAL, -1)
    assert np.isnan(O[100 + 256:]).all() and np.isnan(L[:, 100 + 256:]).all()
    Or, Lr = attention_varlen_ref(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]), x["cu_q"],
                                  x["cu_k"], 0.125, MASK_CAUSAL)
    ok = np.r_[0:356]
    assert np.abs(O[ok] - Or[ok]).max() <= 1e-2 and np.abs(L[:, ok] - Lr[:, ok]).max() <= 1e-3


@pytest.mark.parametrize("d", [32, 96, 256])
def test_extra_head_dims_self_attention(d):
    import torch

    import exact_attention_92_amd as fa
    for N in (1, 65, 300, 1000):
        x = make_raw(2, 3, N, d, "bf16", seed=240 + N + d, q_mult=2.0,
                     kv_len_range=(max(1, N // 3), N))
        for mask in (MASK_NONE, MASK_CAUSAL, MASK_KEY_PADDING, MASK_CAUSAL | MASK_KEY_PADDING):
            q, k, v = (to_dev(x[t]) for t in "qkv")
            o = torch.full_like(q, float("nan"))
            lse = torch.full((2, 3, N), float("nan"), device="cuda")
            fa.fa_fwd(q, k, v, o, lse, d ** -0.5, mask, torch.from_numpy(x["kv_lens"]).cuda())
            torch.cuda.synchronize()
            ref = attention_general_ref(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]),
                                        d ** -0.5, mask, -1, x["kv_lens"], magnitudes=True)
            compare_bound(o_to_f64(o), lse.cpu().numpy().astype(np.float64), ref,
                          f"fa_fwd d={d} N={N} mask={mask}")


@pytest.mark.parametrize("d", [32, 96, 256])
def test_extra_head_dims_general(d):
    import torch

    import exact_attention_92_amd as fa
    for Nq, Nk in ((77, 300), (300, 129)):
        xq = make_raw(2, 2, Nq, d, "bf16", seed=250 + Nq + d, q_mult=2.0)
        xk = make_raw(2, 2, Nk, d, "bf16", seed=251 + Nk + d)
        for mask, window in ((MASK_CAUSAL, -1), (MASK_CAUSAL, 17), (MASK_NONE, 40)):
            q = to_dev(xq["q"]).permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
            k, v = to_dev(xk["k"]), to_dev(xk["v"])
            o = torch.full((2, 2, Nq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
            lse = torch.full((2, 2, Nq), float("nan"), device="cuda")
            fa.fa_fwd_general(q, k, v, o, lse, d ** -0.5, mask, window)
            torch.cuda.synchronize()
            ref = attention_general_ref(to_f64(xq["q"]), to_f64(xk["k"]), to_f64(xk["v"]),
                                        d ** -0.5, mask, window, magnitudes=True)
            compare_bound(o_to_f64(o), lse.cpu().numpy().astype(np.float64), ref,
                          f"general d={d} Nq={Nq} Nk={Nk} mask={mask} W={window}")


def test_varlen_bench_workload_sampled_sequences():
    """The packed bench workload at full size, in the launch the bench times;
    three of its sequences (the longest among them) checked in full."""
    from fa_inputs import GENERAL_WORKLOADS, make_inputs
    wl = GENERAL_WORKLOADS["bf16_varlen_b16h32_n512_4096_d128_causal"]
    say(f"[varlen] {wl.name}")
    x = make_inputs(wl)
    O, L = run_varlen(x, wl.N, wl.scale, wl.mask_kind, wl.window_left)
    cu = x["cu_q"]
    for s_ in (0, 1, wl.B - 1):
        rows = slice(int(cu[s_]), int(cu[s_ + 1]))
        sub_cu = np.array([0, cu[s_ + 1] - cu[s_]], dtype=np.int32)
        ref = attention_varlen_ref(to_f64(x["q"][rows]), to_f64(x["k"][rows]),
                                   to_f64(x["v"][rows]), sub_cu, sub_cu, wl.scale, wl.mask_kind,
                                   wl.window_left, magnitudes=True)
        t = (1, 0, 2)
        compare_bound(O[rows].transpose(t), L[:, rows], (ref[0].transpose(t), ref[1],
                                                         ref[2].transpose(t)),
                      f"{wl.name} sequence {s_} (n={sub_cu[1]})")
    assert not np.isnan(O).any() and not np.isnan(L).any()


def test_head_dim_256_long_causal_sampled_rows():
    """d = 256 at N = 8192 (64 key blocks per row block), sampled rows."""
    import torch

    import exact_attention_92_amd as fa
    B, H, N, d = 1, 4, 8192, 256
    x = make_raw(B, H, N, d, "bf16", seed=260, q_mult=2.0)
    say(f"[d=256] N={N} causal")
    q, k, v = (to_dev(x[t]) for t in "qkv")
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    fa.fa_fwd(q, k, v, o, lse, d ** -0.5, MASK_CAUSAL)
    torch.cuda.synchronize()
    O, L = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    rows = np.unique(np.r_[0:40, np.linspace(0, N - 1, 40).astype(int), N - 40:N])
    ref = attention_general_ref(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]), d ** -0.5,
                                MASK_CAUSAL, -1, magnitudes=True, rows=rows)
    assert not np.isnan(O).any() and not np.isnan(L).any()
    compare_bound(O[:, :, rows], L[:, :, rows], ref, f"d=256 N={N} causal sampled")
