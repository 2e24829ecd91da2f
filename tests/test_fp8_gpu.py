"""GPU parity of the FP8 (E4M3) forward against the CPU oracle.

The oracle computes exact attention of the dequantized E4M3 values (the same
bytes and scales the kernel reads).  The kernel's errors, per query row r and
head dimension t:

* Logits.  The E4M3 matrix cores do not accumulate exactly in fp32: over
  random E4M3 operands the error of a 64-deep product measured at most
  2^-11.1 of its largest |term| -- the precision of the FP16 accumulation
  the FP8 path of "FlashAttention 完整解析" (§5.5) describes.  So each logit
  is off by at most g_r = 2^-11 |scale| sum_t |q_rt k_ct|, bounded here by
  2^-11 |scale| |q_r|_2 max_c |k_c|_2 (Cauchy-Schwarz).  That moves every
  p_rc and the row sum by a factor within e^(+-g_r), so O by at most
  (e^(2 g_r) - 1) (P |V|)_rt, and LSE by at most g_r.
* P.  The kernel's reference max lags the row max by at most 2^2 (binary
  orders of headroom, so p <= 4), and 448 p / 4 is rounded to E4M3: relative
  error at most 2^-4 for normal values, absolute at most 2^-10 (half the
  smallest subnormal step) below 2^-6, i.e. 2^-10 * 4 / 448 in p; the
  normalisation divides by the fp32 sum of the unrounded p.  Summed over the
  visible keys this gives 2^-4 (P |V|)_rt + 2^-8/448 (sum_J |v_t|)_r / l_r.
* O's own bf16 rounding: 2^-8 |O_ref|; fp32 sums and exp2: 1e-5 (P |V|).

LSE: the logit term plus 1e-3 (the bf16 path's bar for its fp32 sums).
Each named workload also keeps relative Frobenius <= 5e-2.  Outputs are
pre-filled with NaN so an unwritten element fails.
"""
import numpy as np
import pytest

from fa_inputs import (FP8_WORKLOADS, MASK_CAUSAL, MASK_KEY_PADDING, MASK_NONE, inputs_f64,
                       make_inputs, make_raw)
from gpu_util import o_to_f64, say
from oracle import attention_ref

pytestmark = pytest.mark.gpu

MASKS = [MASK_NONE, MASK_CAUSAL, MASK_KEY_PADDING, MASK_CAUSAL | MASK_KEY_PADDING]
U8, SUB, U16, NOISE = 2.0 ** -4, 2.0 ** -10 * 4 / 448.0, 2.0 ** -8, 1e-5
ACC = 2.0 ** -11     # accumulation error of the E4M3 matrix cores, per |term|


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")
    import exact_attention_92_amd as fa
    fa.load_library()


def run_fp8(x, scale, mask):
    import torch

    import exact_attention_92_amd as fa
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, k, v = (dev(x[n]) for n in "qkv")
    qs, ks, vs = (dev(x[n + "_descale"]) for n in "qkv")
    kv = None if x.get("kv_lens") is None else dev(np.asarray(x["kv_lens"], dtype=np.int32))
    B, H, N, d = q.shape
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    fa.fa_fwd_fp8(q, k, v, qs, ks, vs, o, lse, scale, mask, kv)
    torch.cuda.synchronize()
    return o_to_f64(o), lse.cpu().numpy().astype(np.float64)


def oracle(x, scale, mask, rows=None):
    """fp64 O, LSE, magnitudes, and the per-row logit error bound g_r."""
    q, k, v = inputs_f64(x)
    O, L, M = attention_ref(q, k, v, scale, mask, x.get("kv_lens"), rows=rows, workers=16,
                            magnitudes=True)
    qn = np.linalg.norm(q, axis=3)
    if rows is not None:
        qn = qn[:, :, rows]
    kmax = np.linalg.norm(k, axis=3).max(axis=2)
    g = ACC * abs(float(np.float32(scale))) * qn * kmax[:, :, None]
    return O, L, M, g


def compare_fp8(O, L, ref, what, bulk=False):
    Or, Lr, M, g = ref
    assert not np.isnan(O).any() and not np.isnan(L).any(), f"{what}: unwritten elements"
    empty = ~np.isfinite(Lr)
    assert np.array_equal(~np.isfinite(L), empty), f"{what}: LSE -inf pattern"
    if empty.any():
        assert np.all(L[empty] == -np.inf) and np.all(O[empty] == 0.0), f"{what}: empty rows"
    err = np.abs(O - Or)
    bound = ((U8 + np.expm1(2 * g)[..., None] + NOISE) * M["pv"] + SUB * M["v_over_l"]
             + U16 * np.abs(Or))
    zero = bound == 0
    assert np.all(err[zero] == 0.0), f"{what}: elements with no terms must be 0"
    ratio = float(np.max(err[~zero] / bound[~zero], initial=0.0))
    nrm = np.linalg.norm(Or)
    relf = float(np.linalg.norm(O - Or) / nrm) if nrm > 0 else 0.0
    lse_err = float(np.abs(L[~empty] - Lr[~empty]).max(initial=0.0))
    lse_ratio = float(np.max(np.abs(L[~empty] - Lr[~empty]) / (1e-3 + g[~empty]), initial=0.0))
    say(f"  {what}: relF={relf:.2e} err/bound={ratio:.2f} max|dLSE|={lse_err:.2e} "
        f"(of bound {lse_ratio:.2f})")
    assert ratio <= 1.0, (what, "element bound", ratio)
    assert lse_ratio <= 1.0, (what, "LSE", lse_err)
    if bulk:
        assert relf <= 5e-2, (what, "relative Frobenius", relf)


def test_bench_workload_full_parity():
    wl = FP8_WORKLOADS["fp8_b2h32_n4096_d128_causal"]
    say(f"[fp8 parity] {wl.name}")
    x = make_inputs(wl)
    O, L = run_fp8(x, wl.scale, wl.mask_kind)
    compare_fp8(O, L, oracle(x, wl.scale, wl.mask_kind), wl.name, bulk=True)


@pytest.mark.parametrize("mask", MASKS)
def test_d64_workload_shapes(mask):
    x = make_raw(4, 8, 1024, 64, "fp8", seed=12, kv_len_range=(512, 1024))
    O, L = run_fp8(x, 0.125, mask)
    compare_fp8(O, L, oracle(x, 0.125, mask), f"B4 H8 N1024 d64 mask={mask}", bulk=True)


@pytest.mark.parametrize("d", [64, 128])
def test_causal_items_all_resident(d):
    """B*H = 64 causal heads of 1024 rows: every work item fits on the chip at
    once, so the work order visits 8 heads per XCD group (the head-group
    rule's second branch), not 4."""
    x = make_raw(4, 16, 1024, d, "fp8", seed=4160 + d, q_mult=2.0)
    O, L = run_fp8(x, d ** -0.5, MASK_CAUSAL)
    compare_fp8(O, L, oracle(x, d ** -0.5, MASK_CAUSAL), f"B4 H16 N1024 d{d} causal", bulk=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 4, 63, 65, 127, 129, 1000])
def test_ragged_lengths_all_masks(d, N):
    x = make_raw(2, 3, N, d, "fp8", seed=3000 + N + d, q_mult=2.0,
                 kv_len_range=(max(0, N // 2 - 3), N))
    for mask in MASKS:
        O, L = run_fp8(x, d ** -0.5, mask)
        compare_fp8(O, L, oracle(x, d ** -0.5, mask),
                    f"N={N} d={d} mask={mask} kv={x['kv_lens'].tolist()}")


def test_kv_len_edges():
    N, d = 300, 128
    lens = [0, 1, 63, 64, 65, 127, 128, 129, N]
    x = make_raw(len(lens), 2, N, d, "fp8", seed=79)
    x["kv_lens"] = np.array(lens, dtype=np.int32)
    for mask in (MASK_KEY_PADDING, MASK_KEY_PADDING | MASK_CAUSAL):
        O, L = run_fp8(x, d ** -0.5, mask)
        compare_fp8(O, L, oracle(x, d ** -0.5, mask), f"kv_len edges mask={mask}")


@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.0])
def test_unusual_scales(scale):
    x = make_raw(1, 2, 190, 64, "fp8", seed=11)
    for mask in (MASK_NONE, MASK_CAUSAL):
        O, L = run_fp8(x, scale, mask)
        compare_fp8(O, L, oracle(x, scale, mask), f"scale={scale} mask={mask}")


def test_q_zero_closed_form_long_causal():
    """Q = 0: every probability is exactly 1 (448 / 4 is exact in E4M3), so O_r is
    the mean of the visible V rows up to bf16 rounding, at N = 65536."""
    B, H, N, d = 1, 2, 65536, 128
    say(f"[fp8 closed form] Q=0 causal N={N}")
    x = make_raw(B, H, N, d, "fp8", seed=32)
    x["q"] = np.zeros_like(x["q"])
    O, L = run_fp8(x, d ** -0.5, MASK_CAUSAL)
    _, _, v = inputs_f64(x)
    cnt = np.arange(1, N + 1, dtype=np.float64)
    Or = np.cumsum(v, axis=2) / cnt[None, None, :, None]
    assert np.all(np.abs(O - Or) <= U16 * np.abs(Or) + 1e-5 * np.abs(v).max())
    assert np.max(np.abs(L - np.log(cnt)[None, None, :])) <= 1e-3


def test_hidden_keys_may_hold_nan_codes():
    N, d = 200, 64
    x = make_raw(2, 2, N, d, "fp8", seed=7)
    x["kv_lens"] = np.array([70, 131], dtype=np.int32)
    y = dict(x)
    y["k"], y["v"] = x["k"].copy(), x["v"].copy()
    for b, kl in enumerate(x["kv_lens"]):
        y["k"][b, :, kl:] = 0x7F   # E4M3 NaN
        y["v"][b, :, kl:] = 0xFF
    Oa, La = run_fp8(x, 0.125, MASK_KEY_PADDING)
    Ob, Lb = run_fp8(y, 0.125, MASK_KEY_PADDING)
    assert np.array_equal(Oa, Ob) and np.array_equal(La, Lb)


def test_bitwise_deterministic():
    x = make_raw(2, 8, 1000, 128, "fp8", seed=13)
    runs = [run_fp8(x, 128 ** -0.5, MASK_CAUSAL) for _ in range(3)]
    for O, L in runs[1:]:
        assert np.array_equal(O, runs[0][0]) and np.array_equal(L, runs[0][1])


def test_errors_write_nothing():
    import torch

    import exact_attention_92_amd as fa
    q = torch.zeros((1, 1, 64, 96), dtype=torch.uint8, device="cuda")
    ds = torch.ones((1, 1), dtype=torch.float32, device="cuda")
    o = torch.full((1, 1, 64, 96), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((1, 1, 64), float("nan"), device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_fp8(q, q, q, ds, ds, ds, o, lse, 0.1)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all() and torch.isnan(lse).all()


FP8_EDGES = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 383, 511, 513]


@pytest.mark.parametrize("chunk", range(3))
def test_random_shapes_masks_and_scales(chunk):
    """Seeded random cases: each draws d, B, H, N (half of them at the 64-,
    128- and 256-row block edges), the mask, the key lengths and the scale
    from its own seed, so a failure names a reproducible case."""
    for seed in range(700 + 12 * chunk, 700 + 12 * chunk + 12):
        rng = np.random.default_rng(seed)
        d = int(rng.choice([64, 128]))
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 6))
        N = int(rng.choice(FP8_EDGES)) if rng.random() < 0.5 else int(rng.integers(1, 1200))
        mask = int(rng.integers(0, 4))
        scale = float(d ** -0.5 * rng.choice([1.0, 1.0, -0.7, 2.5]))
        kv_range = (0, N) if mask & MASK_KEY_PADDING else None
        what = f"seed={seed} B={B} H={H} N={N} d={d} mask={mask} scale={scale:.4f}"
        say(what)
        x = make_raw(B, H, N, d, "fp8", seed=seed, q_mult=2.0, kv_len_range=kv_range)
        O, L = run_fp8(x, scale, mask)
        compare_fp8(O, L, oracle(x, scale, mask), what)


@pytest.mark.parametrize("B,H,N,d,mask", [
    (4, 37, 1100, 128, MASK_KEY_PADDING | MASK_CAUSAL),   # 8-wave blocks, 8 does not divide B*H
    (2, 48, 1536, 64, MASK_CAUSAL),                       # 8-wave blocks, heads split over XCDs
    (3, 40, 900, 128, MASK_KEY_PADDING),
])
def test_grids_larger_than_the_chip(B, H, N, d, mask):
    """More workgroups than the chip holds at once, with and without a head
    count that divides by the XCD count, on every element."""
    kv_range = (1, N) if mask & MASK_KEY_PADDING else None
    x = make_raw(B, H, N, d, "fp8", seed=B * 100 + H + N + d, q_mult=2.0, kv_len_range=kv_range)
    what = f"B={B} H={H} N={N} d={d} mask={mask}"
    say(what)
    O, L = run_fp8(x, d ** -0.5, mask)
    compare_fp8(O, L, oracle(x, d ** -0.5, mask), what, bulk=True)


def test_largest_n():
    """N at the entry point's bound ((N + 256) d 4 <= 2^32 - 1) with key
    padding to 200 keys: sampled rows through the last block against the
    oracle, every output written, one row more refused.  Inputs are drawn
    on the device; the sampled query rows are placed first in a 200-row
    query block for the oracle (unmasked rows are independent)."""
    import torch

    import exact_attention_92_amd as fa
    d, KV = 128, 200
    N = (2 ** 32 - 1) // (d * 4) - 256
    assert (N + 257) * d * 4 > 2 ** 32 - 1
    say(f"[fp8 largest N] N={N} d={d} key padding {KV}")
    g = torch.Generator(device="cuda").manual_seed(31)
    q, k, v = (torch.randn((1, 1, N, d), generator=g, device="cuda").to(torch.float8_e4m3fn)
               .view(torch.uint8) for _ in range(3))
    ds = torch.ones((1, 1), device="cuda")
    o = torch.full((1, 1, N, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((1, 1, N), float("nan"), device="cuda")
    kv = torch.tensor([KV], dtype=torch.int32, device="cuda")
    scale = d ** -0.5
    fa.fa_fwd_fp8(q, k, v, ds, ds, ds, o, lse, scale, MASK_KEY_PADDING, kv)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any().item() and torch.isfinite(lse).all().item()
    rows = np.array(sorted({0, 1, 127, 128, 255, 256, N // 2, N - 257, N - 256, N - 129, N - 128,
                            N - 65, N - 2, N - 1}))
    qs = np.zeros((1, 1, KV, d), dtype=np.uint8)
    qs[:, :, :len(rows)] = q[:, :, rows].cpu().numpy()
    one = np.ones((1, 1), dtype=np.float32)
    x = {"q": qs, "k": k[:, :, :KV].cpu().numpy(), "v": v[:, :, :KV].cpu().numpy(),
         "kv_lens": None, "q_descale": one, "k_descale": one, "v_descale": one}
    ref = oracle(x, scale, MASK_NONE, rows=np.arange(len(rows)))
    O = o_to_f64(o[:, :, rows])
    L = lse[:, :, rows].cpu().numpy().astype(np.float64)
    st = fa.load_library().fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), ds.data_ptr(),
                                      ds.data_ptr(), ds.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                      1, 1, N + 1, d, scale, MASK_KEY_PADDING, kv.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_ERR_INVALID_ARG
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    compare_fp8(O, L, ref, f"largest N={N}")
