"""GPU parity of paged-KV decode against the CPU oracle.

The kernels keep every probability and sum in fp32 (nothing is rounded to
bf16 before the end), so per element the error is O's own bf16 rounding plus
fp32 noise:  |O - O_ref| <= 2^-8 |O_ref| + 1e-5 (P |V|);  LSE within 2e-4.
Requests with no cached token must give O = 0 and LSE = -inf exactly.
Outputs are pre-filled with NaN so an unwritten element fails.
"""
import numpy as np
import pytest

from fa_inputs import DECODE_WORKLOADS, bf16_bits_to_f32, make_paged_decode
from gpu_util import say
from oracle.paged_decode_ref import paged_decode_ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")
    import exact_attention_92_amd as fa
    fa.load_library()


def run_decode(x, scale):
    import torch

    import exact_attention_92_amd as fa

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    q, kp, vp = bf(x["q"]), bf(x["k_pool"]), bf(x["v_pool"])
    tab = torch.from_numpy(x["block_tables"]).cuda()
    lens = torch.from_numpy(x["seq_lens"]).cuda()
    B, H, d = q.shape
    o = torch.full((B, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H), float("nan"), device="cuda")
    need = fa.fa_decode_paged_workspace_bytes(B, H, d, kp.shape[2], tab.shape[1])
    ws = torch.full(((need + 3) // 4,), float("nan"), device="cuda")
    fa.fa_decode_paged(q, kp, vp, tab, lens, o, lse, ws, scale)
    torch.cuda.synchronize()
    return (o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))


def oracle(x, scale):
    f = bf16_bits_to_f32
    return paged_decode_ref(f(x["q"]), f(x["k_pool"]), f(x["v_pool"]), x["block_tables"],
                            x["seq_lens"], scale, magnitudes=True)


def compare(O, L, ref, what):
    Or, Lr, M = ref
    assert not np.isnan(O).any() and not np.isnan(L).any(), f"{what}: unwritten"
    empty = ~np.isfinite(Lr)
    assert np.array_equal(~np.isfinite(L), empty), what
    assert np.all(O[empty] == 0.0) and np.all(L[empty] == -np.inf), what
    err = np.abs(O - Or)
    bound = 2.0 ** -8 * np.abs(Or) + 1e-5 * M
    ratio = float(np.max(err / np.where(bound > 0, bound, np.inf), initial=0.0))
    lerr = float(np.abs(L[~empty] - Lr[~empty]).max(initial=0.0))
    say(f"  {what}: err/bound={ratio:.2f} max|dLSE|={lerr:.2e}")
    assert np.all(err[bound == 0] == 0.0), what
    assert ratio <= 1.0 and lerr <= 2e-4, (what, ratio, lerr)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bs", [8, 16, 64, 256])
def test_block_sizes_and_lengths(d, bs):
    lens = np.random.default_rng(bs + d).integers(0, 1500, size=6)
    lens[:4] = [0, 1, bs, 512 + bs + 3]
    x = make_paged_decode(6, 3, d, bs, (0, 1500), seed=100 + bs + d, spare=5, lens=lens)
    O, L = run_decode(x, d ** -0.5)
    compare(O, L, oracle(x, d ** -0.5), f"d={d} bs={bs} lens={x['seq_lens'].tolist()}")


def test_bench_workload_sampled_requests():
    wl = DECODE_WORKLOADS["decode_b32h32_d128_bs64_len1k8k"]
    say(f"[decode parity] {wl.name}")
    x = make_paged_decode(wl.B, wl.H, wl.d, wl.block_size, wl.len_range, wl.seed, wl.spare)
    O, L = run_decode(x, wl.scale)
    pick = [0, 7, 13, 31]
    sub = dict(x, q=x["q"][pick], block_tables=x["block_tables"][pick], seq_lens=x["seq_lens"][pick])
    compare(O[pick], L[pick], oracle(sub, wl.scale), wl.name + " (4 requests)")


def test_unused_slots_and_spare_blocks_may_hold_nan():
    x = make_paged_decode(4, 2, 128, 64, (100, 700), seed=55, spare=3)
    y = {k: v.copy() for k, v in x.items()}
    bs = 64
    used = set()
    for b, n in enumerate(x["seq_lens"]):
        nb = (int(n) + bs - 1) // bs
        used.update(int(t) for t in x["block_tables"][b, :nb])
        last = int(x["block_tables"][b, nb - 1])
        tail = int(n) - (nb - 1) * bs
        y["k_pool"][last, :, tail:] = 0x7FC0
        y["v_pool"][last, :, tail:] = 0x7FC0
    spare = [i for i in range(x["k_pool"].shape[0]) if i not in used]
    y["k_pool"][spare] = 0x7FC0
    y["v_pool"][spare] = 0x7FC0
    Oa, La = run_decode(x, 0.1)
    Ob, Lb = run_decode(y, 0.1)
    assert np.array_equal(Oa, Ob) and np.array_equal(La, Lb)


@pytest.mark.parametrize("scale", [-0.5, 0.0, 1.5])
def test_unusual_scales(scale):
    x = make_paged_decode(3, 2, 64, 16, (1, 900), seed=56)
    O, L = run_decode(x, scale)
    compare(O, L, oracle(x, scale), f"scale={scale}")


def test_q_zero_long_sequence_closed_form():
    x = make_paged_decode(2, 2, 128, 64, (60000, 65536), seed=57)
    x["q"] = np.zeros_like(x["q"])
    O, L = run_decode(x, 0.1)
    v = bf16_bits_to_f32(x["v_pool"])
    for b in range(2):
        n = int(x["seq_lens"][b])
        nb = (n + 63) // 64
        for h in range(2):
            V = np.concatenate([v[int(t), h] for t in x["block_tables"][b, :nb]])[:n]
            want = V.astype(np.float64).mean(axis=0)
            assert np.all(np.abs(O[b, h] - want) <= 2.0 ** -8 * np.abs(want) + 1e-6)
            assert abs(L[b, h] - np.log(n)) <= 2e-4


def test_deterministic_and_errors_write_nothing():
    import torch

    import exact_attention_92_amd as fa
    x = make_paged_decode(3, 2, 128, 32, (1, 2000), seed=58)
    a = run_decode(x, 0.2)
    b = run_decode(x, 0.2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    q = torch.zeros((1, 1, 96), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((1, 1, 8, 96), dtype=torch.bfloat16, device="cuda")
    tab = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    lens = torch.ones((1,), dtype=torch.int32, device="cuda")
    o = torch.full((1, 1, 96), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((1, 1), float("nan"), device="cuda")
    ws = torch.zeros((1024,), device="cuda")
    with pytest.raises(fa.FaError):
        fa.fa_decode_paged(q, pool, pool, tab, lens, o, lse, ws, 0.1)
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all() and torch.isnan(lse).all()
    assert fa.fa_decode_paged_workspace_bytes(2, 3, 128, 64, 10) == 2 * 3 * 2 * 130 * 4


@pytest.mark.parametrize("B,H,bs,hi", [(65535, 2, 16, 40), (1, 65535, 8, 20)])
def test_largest_batch_and_head_counts(B, H, bs, hi):
    """The request and head counts at their bound (65535, a launch grid
    dimension each), short cached lengths including 0; every output written,
    sampled requests (the first and last included) against the oracle."""
    what = f"decode B={B} H={H} d=64 bs={bs} lengths 0..{hi}"
    say(what)
    x = make_paged_decode(B, H, 64, bs, (0, hi), seed=B + H, spare=2)
    O, L = run_decode(x, 0.125)
    assert not np.isnan(O).any() and not np.isnan(L).any(), f"{what}: unwritten"
    sub = np.unique(np.r_[0:3, B - 3:B, np.random.default_rng(5).integers(0, B, 60)])
    sub = sub[(sub >= 0) & (sub < B)]
    f = bf16_bits_to_f32
    ref = paged_decode_ref(f(x["q"][sub]), f(x["k_pool"]), f(x["v_pool"]),
                           x["block_tables"][sub], x["seq_lens"][sub], 0.125, magnitudes=True)
    compare(O[sub], L[sub], ref, what)
