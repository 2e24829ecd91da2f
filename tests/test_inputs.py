"""The seeded input generator: reproducible, correctly encoded, right shapes."""
import numpy as np
import pytest

from fa_inputs import (MASK_CAUSAL, MASK_KEY_PADDING, WORKLOADS, bf16_bits_to_f32,
                       f32_to_bf16_bits, make_inputs, make_raw, to_f64)


def test_reproducible_from_seed():
    a = make_raw(1, 2, 33, 8, "bf16", seed=7, kv_len_range=(3, 9))
    b = make_raw(1, 2, 33, 8, "bf16", seed=7, kv_len_range=(3, 9))
    c = make_raw(1, 2, 33, 8, "bf16", seed=8, kv_len_range=(3, 9))
    for n in "qkv":
        assert np.array_equal(a[n], b[n])
        assert not np.array_equal(a[n], c[n])
    assert np.array_equal(a["kv_lens"], b["kv_lens"])


def test_bf16_rne_matches_torch():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3e38, -3e38,
                                  1e-40, np.inf, -np.inf], dtype=np.float32)])
    ours = f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    # Ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7.
    assert f32_to_bf16_bits(np.array([1.00390625], np.float32))[0] == 0x3F80
    assert np.array_equal(bf16_bits_to_f32(ours[:100]).view(np.uint32) >> 16, ours[:100])


def test_workload_shapes_and_recipe():
    wl = WORKLOADS["bf16_b8h16_n2048_d64_keypad"]
    x = make_inputs(wl)
    assert x["q"].shape == (8, 16, 2048, 64) and x["q"].dtype == np.uint16
    assert x["kv_lens"].dtype == np.int32 and x["kv_lens"].shape == (8,)
    assert ((x["kv_lens"] >= 1024) & (x["kv_lens"] <= 2048)).all()
    assert wl.mask_kind == MASK_KEY_PADDING
    f = WORKLOADS["f32_b1h1_n256_d64"]
    y = make_inputs(f)
    assert y["q"].dtype == np.float32 and y["kv_lens"] is None
    assert abs(f.scale - 0.125) == 0.0


def test_q_multiplier_is_exact():
    a = make_raw(1, 1, 64, 16, "f32", seed=3, q_mult=1.0)
    b = make_raw(1, 1, 64, 16, "f32", seed=3, q_mult=2.0)
    assert np.array_equal(b["q"], a["q"] * 2)
    assert np.array_equal(b["k"], a["k"])


def test_flop_formula():
    wl = WORKLOADS["bf16_b2h32_n4096_d128_causal"]
    assert wl.mask_kind == MASK_CAUSAL
    assert wl.flops() == 4 * 2 * 32 * 4096 * 4096 * 128 / 2
    assert abs(wl.scale - 1 / np.sqrt(128)) < 1e-8
    assert to_f64(np.array([0x3F80], np.uint16))[0] == 1.0


def test_grad_out_stream_leaves_forward_inputs_unchanged():
    """dO comes from a fifth child seed; Q, K, V keep their streams."""
    from fa_inputs import make_bwd_inputs, make_grad_out
    wl = WORKLOADS["bf16_b4h16_n1024_d64_causal"]
    x = make_inputs(wl)
    y = make_bwd_inputs(wl)
    for n in "qkv":
        assert np.array_equal(x[n], y[n])
    assert y["do"].shape == x["q"].shape and y["do"].dtype == np.uint16
    assert np.array_equal(y["do"], make_grad_out(wl.B, wl.H, wl.N, wl.d, "bf16", wl.seed))
    assert not np.array_equal(y["do"], y["q"])
    f = make_grad_out(1, 2, 8, 4, "f32", 3)
    assert f.dtype == np.float32 and abs(float(f.mean())) < 1.0


def test_fp8_e4m3_encoding_matches_torch():
    """Every float32 that rounds to each code, the ties between codes, the
    subnormals and the clamp at 448 agree with torch's float8_e4m3fn."""
    torch = pytest.importorskip("torch")
    from fa_inputs import FP8_MAX, f32_to_fp8_e4m3, fp8_e4m3_to_f64
    codes = np.arange(256, dtype=np.uint8)
    vals = fp8_e4m3_to_f64(codes)
    fin = np.isfinite(vals)
    assert np.nanmax(vals) == FP8_MAX and np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    # Round trip of every finite code (negative zero keeps its sign bit).
    assert np.array_equal(f32_to_fp8_e4m3(vals[fin]), codes[fin])
    pos = np.sort(vals[(vals >= 0) & fin])
    mids = (pos[1:] + pos[:-1]) / 2
    g = np.random.default_rng(0)
    x = np.concatenate([pos, mids, -mids, np.nextafter(mids.astype(np.float32), 0),
                        np.nextafter(mids.astype(np.float32), 1000),
                        g.standard_normal(20000) * 40, g.standard_normal(2000) * 1e-3,
                        [447.9, 448.0, 460.0, 463.99, -448.0]]).astype(np.float32)
    want = torch.from_numpy(np.clip(x, -FP8_MAX, FP8_MAX)).to(torch.float8_e4m3fn)
    assert np.array_equal(f32_to_fp8_e4m3(x), want.view(torch.uint8).numpy())
    assert np.array_equal(fp8_e4m3_to_f64(want.view(torch.uint8).numpy()),
                          want.to(torch.float64).numpy())


def test_fp8_per_head_quantization_recipe():
    from fa_inputs import FP8_WORKLOADS, inputs_f64, make_inputs, make_raw
    wl = FP8_WORKLOADS["fp8_b2h32_n4096_d128_causal"]
    x = make_raw(2, 3, 64, 64, "fp8", seed=3, q_mult=2.0)
    ref = make_raw(2, 3, 64, 64, "f32", seed=3, q_mult=2.0)
    q, k, v = inputs_f64(x)
    for name, deq in zip("qkv", (q, k, v)):
        ds = x[name + "_descale"]
        assert ds.shape == (2, 3) and ds.dtype == np.float32
        amax = np.abs(ref[name]).max(axis=(2, 3))
        assert np.allclose(ds, amax / 448.0, rtol=1e-7)
        # Each head uses its full range, and the relative error is within the
        # E4M3 rounding bound (half a step: 2^-4 relative for normal values).
        assert np.max(np.abs(x[name]) & 0x7F) == 0x7E
        err = np.abs(deq - ref[name])
        scale = ds[:, :, None, None].astype(np.float64)
        assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(ref[name]), 2.0 ** -10 * scale) * 1.0001)
    assert wl.dtype == "fp8" and make_inputs(wl)["q"].dtype == np.uint8


def test_fp8_per_tile_quantization_recipe():
    """One E4M3 scale per 128 rows: each tile uses its full range (its largest
    code is 448), each element is within the E4M3 rounding bound of its draw,
    and with a single tile the recipe is the per-head one (same codes and
    scale)."""
    from fa_inputs import (FP8_TILE, inputs_f64, make_raw, make_raw_fp8_tiled,
                           quantize_fp8_per_head, quantize_fp8_per_tile)
    x = make_raw_fp8_tiled(2, 3, 300, 64, seed=5, q_mult=2.0, tile_gain=4.0)
    q, k, v = inputs_f64(x)
    T = -(-300 // FP8_TILE)
    for name, deq in (("q", q), ("k", k)):
        ds, raw = x[name + "_descale"], x[name + "_f32"]
        assert ds.shape == (2, 3, T) and ds.dtype == np.float32
        for t in range(T):
            rows = slice(t * FP8_TILE, min(300, (t + 1) * FP8_TILE))
            amax = np.abs(raw[:, :, rows]).max(axis=(2, 3))
            assert np.allclose(ds[:, :, t], amax / 448.0, rtol=1e-7)
            assert np.all((x[name][:, :, rows] & 0x7F).reshape(2, 3, -1).max(axis=2) == 0x7E)
            err = np.abs(deq[:, :, rows] - raw[:, :, rows])
            step = ds[:, :, t][:, :, None, None].astype(np.float64)
            assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(raw[:, :, rows]),
                                            2.0 ** -10 * step) * 1.0001)
    # the gains really spread the tiles' ranges
    assert np.log2(x["q_descale"].max() / x["q_descale"].min()) > 4
    assert x["v_descale"].shape == (2, 3)
    # one tile: identical to per-head quantization
    y = make_raw(1, 2, 100, 32, "f32", seed=9)["q"]
    ct, st = quantize_fp8_per_tile(y)
    ch, sh = quantize_fp8_per_head(y)
    assert np.array_equal(ct, ch) and np.array_equal(st[:, :, 0], sh)
