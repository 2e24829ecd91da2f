"""GPU parity of the FP8 forward with per-tile Q/K scales (fa_fwd_fp8_tiled).

Block quantization at tile granularity: Q and K carry one scale per 128 rows
of a head, V one per head.  The oracle computes exact attention of the
dequantized values (the same bytes and scales the kernel reads); the error
bounds are those of the per-head FP8 path (tests/test_fp8_gpu.py), which are
stated in terms of the dequantized Q, K and V and so hold unchanged.
"""
import numpy as np
import pytest

from fa_inputs import (MASK_CAUSAL, MASK_KEY_PADDING, MASK_NONE, FP8_TILE, make_raw,
                       make_raw_fp8_tiled, quantize_fp8_per_head)
from gpu_util import o_to_f64, say
from oracle import attention_ref
from test_fp8_gpu import compare_fp8, oracle, run_fp8

pytestmark = pytest.mark.gpu

MASKS = [MASK_NONE, MASK_CAUSAL, MASK_KEY_PADDING, MASK_CAUSAL | MASK_KEY_PADDING]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")
    import exact_attention_92_amd as fa
    fa.load_library()


def run_tiled(x, scale, mask):
    import torch

    import exact_attention_92_amd as fa
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, k, v = (dev(x[n]) for n in "qkv")
    qs, ks, vs = (dev(x[n + "_descale"]) for n in "qkv")
    kv = None if x.get("kv_lens") is None else dev(np.asarray(x["kv_lens"], dtype=np.int32))
    B, H, N, d = q.shape
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    fa.fa_fwd_fp8_tiled(q, k, v, qs, ks, vs, o, lse, scale, mask, kv)
    torch.cuda.synchronize()
    return o_to_f64(o), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("d", [64, 128])
def test_shared_scales_reproduce_the_per_head_path(d):
    """Per-head inputs with every tile scale equal to its head's scale: the
    tiled entry point computes the same logit multipliers, so its output is
    bitwise that of fa_fwd_fp8."""
    N = 1000
    x = make_raw(2, 3, N, d, "fp8", seed=600 + d, q_mult=2.0, kv_len_range=(400, N))
    T = -(-N // FP8_TILE)
    y = dict(x, fp8_tiled=True,
             q_descale=np.repeat(x["q_descale"][:, :, None], T, axis=2),
             k_descale=np.repeat(x["k_descale"][:, :, None], T, axis=2))
    for mask in (MASK_CAUSAL, MASK_CAUSAL | MASK_KEY_PADDING):
        Oh, Lh = run_fp8(x, d ** -0.5, mask)
        Ot, Lt = run_tiled(y, d ** -0.5, mask)
        assert np.array_equal(Oh, Ot) and np.array_equal(Lh, Lt), (d, mask)


def test_bench_shape_tiled_full_parity():
    """B=2 H=32 N=4096 d=128 causal, Q x2, tiles spread over 2^[-3, 3]."""
    x = make_raw_fp8_tiled(2, 32, 4096, 128, seed=3, q_mult=2.0, tile_gain=3.0)
    say("[fp8 tiled parity] B2 H32 N4096 d128 causal")
    O, L = run_tiled(x, 128 ** -0.5, MASK_CAUSAL)
    compare_fp8(O, L, oracle(x, 128 ** -0.5, MASK_CAUSAL), "tiled B2 H32 N4096 d128", bulk=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 127, 129, 300, 1000])
def test_tiled_ragged_all_masks(d, N):
    x = make_raw_fp8_tiled(2, 3, N, d, seed=700 + N + d, q_mult=2.0, tile_gain=4.0,
                           kv_len_range=(max(0, N // 2 - 3), N))
    for mask in MASKS:
        O, L = run_tiled(x, d ** -0.5, mask)
        compare_fp8(O, L, oracle(x, d ** -0.5, mask),
                    f"tiled N={N} d={d} mask={mask} kv={x['kv_lens'].tolist()}")


def test_tiles_keep_the_range_of_ordinary_rows():
    """One outlier tile of Q per head (values 2^16 larger) sets a per-head scale
    so coarse that the other rows fall into E4M3's subnormal range; with one
    scale per tile they keep their precision.  On the rows of the ordinary
    tiles, the tiled result is much closer to the attention of the
    unquantized values than the per-head one (the outlier rows' logits are
    huge and their attention one-hot in both, so they are left out)."""
    from fa_inputs import quantize_fp8_per_tile
    x0 = make_raw_fp8_tiled(1, 8, 2048, 128, seed=11)
    q = x0["q_f32"].copy()
    q[:, :, :FP8_TILE] *= np.float32(2.0 ** 16)
    k = x0["k_f32"]
    scale = 128 ** -0.5
    ref, _ = attention_ref(q.astype(np.float64), k.astype(np.float64),
                           x0["v_f32"].astype(np.float64), scale, MASK_CAUSAL, None, workers=16)
    common = {"v": x0["v"], "v_descale": x0["v_descale"], "kv_lens": None}
    (qt, qst), (kt, kst) = quantize_fp8_per_tile(q), quantize_fp8_per_tile(k)
    Ot, _ = run_tiled(dict(common, q=qt, k=kt, q_descale=qst, k_descale=kst, fp8_tiled=True),
                      scale, MASK_CAUSAL)
    (qh, qsh), (kh, ksh) = quantize_fp8_per_head(q), quantize_fp8_per_head(k)
    Oh, _ = run_fp8(dict(common, q=qh, k=kh, q_descale=qsh, k_descale=ksh), scale, MASK_CAUSAL)
    rows = slice(FP8_TILE, None)
    nrm = np.linalg.norm(ref[:, :, rows])
    et = np.linalg.norm(Ot[:, :, rows] - ref[:, :, rows]) / nrm
    eh = np.linalg.norm(Oh[:, :, rows] - ref[:, :, rows]) / nrm
    say(f"  relF against the unquantized draws (ordinary rows): per tile {et:.3e}, "
        f"per head {eh:.3e}")
    assert et < 0.5 * eh, (et, eh)


def test_tiled_rejects_wrong_scale_counts():
    import torch

    import exact_attention_92_amd as fa
    x = make_raw_fp8_tiled(1, 2, 200, 64, seed=1)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, k, v = (dev(x[n]) for n in "qkv")
    o = torch.empty((1, 2, 200, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 2, 200), dtype=torch.float32, device="cuda")
    per_head = dev(np.ones((1, 2), np.float32))
    with pytest.raises(ValueError):
        fa.fa_fwd_fp8_tiled(q, k, v, per_head, dev(x["k_descale"]), dev(x["v_descale"]), o, lse,
                            0.125)
