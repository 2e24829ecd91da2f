"""Seeded random sweep of the bf16 forward entry points against the oracle.

Each case draws its shape, head dimension, mask, key lengths, window and
layout from a fixed seed (so a failure names a reproducible case) and checks
the GPU result element by element with the bounds of the general-layout tests
(tests/gpu_util.compare_bound): |err| <= 2^-8 |O_ref| + (2^-7 + 1e-5) (P|V|),
relative Frobenius <= 5e-3, LSE within 1e-3, empty rows exactly O = 0 and
LSE = -inf, nothing left unwritten.  Lengths straddle the 64- and 128-key
block edges of the kernels and the 128/256-row query blocks.
"""
import numpy as np
import pytest

from fa_inputs import MASK_KEY_PADDING, make_packed, make_raw, to_f64
from gpu_util import compare_bound, o_to_f64, say, to_dev
from oracle import attention_general_ref, attention_varlen_ref

pytestmark = pytest.mark.gpu


DIMS = [32, 64, 96, 128, 256]
EDGES = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 191, 255, 256, 257, 383, 511, 513]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")
    import exact_attention_92_amd as fa
    fa.load_library()


def _length(rng):
    return int(rng.choice(EDGES)) if rng.random() < 0.5 else int(rng.integers(1, 700))


def _case(seed):
    rng = np.random.default_rng(seed)
    d = int(rng.choice(DIMS))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    Nq = _length(rng)
    Nk = Nq if rng.random() < 0.4 else _length(rng)
    mask = int(rng.integers(0, 4))
    window = -1 if rng.random() < 0.5 else int(rng.choice([0, 1, 17, 64, 127, 200]))
    layout = "bnhd" if rng.random() < 0.3 else "bhnd"
    scale = float(d ** -0.5 * rng.choice([1.0, 1.0, 1.0, -0.7, 2.5]))
    kv_range = (0, Nk) if mask & MASK_KEY_PADDING else None
    xq = make_raw(B, H, Nq, d, "bf16", seed=1000 + seed, q_mult=2.0)
    xk = make_raw(B, H, Nk, d, "bf16", seed=2000 + seed, kv_len_range=kv_range)
    x = {"q": xq["q"], "k": xk["k"], "v": xk["v"], "kv_lens": xk["kv_lens"]}
    return x, d, B, H, Nq, Nk, mask, window, layout, scale


def _run(x, scale, mask, window, layout, self_attention):
    import torch

    import exact_attention_92_amd as fa

    def dev(a):
        t = to_dev(a)
        if layout == "bnhd":
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
    if self_attention:
        fa.fa_fwd(q, k, v, o, lse, scale, mask, kv)
    else:
        fa.fa_fwd_general(q, k, v, o, lse, scale, mask, window, kv)
    torch.cuda.synchronize()
    return o_to_f64(o.contiguous()), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("chunk", range(10))
def test_random_general_and_self_attention(chunk):
    for seed in range(20 * chunk, 20 * chunk + 20):
        x, d, B, H, Nq, Nk, mask, window, layout, scale = _case(seed)
        self_attn = Nq == Nk and window == -1 and layout == "bhnd"
        what = (f"seed={seed} {'fa_fwd' if self_attn else 'fa_fwd_general'} B={B} H={H} "
                f"Nq={Nq} Nk={Nk} d={d} mask={mask} W={window} {layout} scale={scale:.4f}")
        say(what)
        O, L = _run(x, scale, mask, window, layout, self_attn)
        ref = attention_general_ref(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]), scale, mask,
                                    window, x.get("kv_lens"), magnitudes=True)
        compare_bound(O, L, ref, what)


@pytest.mark.parametrize("chunk", range(4))
def test_random_packed_sequences(chunk):
    import torch

    import exact_attention_92_amd as fa
    for seed in range(500 + 10 * chunk, 500 + 10 * chunk + 10):
        rng = np.random.default_rng(seed)
        d = int(rng.choice(DIMS))
        H = int(rng.integers(1, 4))
        nseq = int(rng.integers(1, 6))
        lq = [_length(rng) if rng.random() < 0.8 else 0 for _ in range(nseq)]
        lk = [q + int(rng.integers(0, 200)) if rng.random() < 0.7 else _length(rng) for q in lq]
        mask = int(rng.integers(0, 2))
        window = -1 if rng.random() < 0.5 else int(rng.choice([0, 17, 128, 300]))
        what = f"seed={seed} fa_fwd_varlen H={H} d={d} lq={lq} lk={lk} mask={mask} W={window}"
        say(what)
        x = make_packed(lq, lk, H, d, seed=seed, q_mult=2.0)
        cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
        cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
        tq = int(cu_q[-1])
        if tq == 0:
            continue
        q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
        o = torch.full((tq, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((H, tq), float("nan"), device="cuda")
        scale = d ** -0.5
        fa.fa_fwd_varlen(q, k, v, o, lse, torch.from_numpy(cu_q).cuda(),
                         torch.from_numpy(cu_k).cuda(), max(lq), scale, mask, window)
        torch.cuda.synchronize()
        Or, Lr, M = attention_varlen_ref(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]), cu_q,
                                         cu_k, scale, mask, window, magnitudes=True)
        O = o_to_f64(o)                               # [tq, H, d]
        L = lse.cpu().numpy().astype(np.float64)      # [H, tq]
        compare_bound(O.transpose(1, 0, 2), L, (Or.transpose(1, 0, 2), Lr, M.transpose(1, 0, 2)),
                      what)


@pytest.mark.parametrize("B,H,N,d,mask", [
    (3, 37, 1000, 64, MASK_KEY_PADDING | 1),   # 888 work items > resident: looping, fallback order
    (5, 29, 700, 32, MASK_KEY_PADDING),        # B*H not a multiple of 8
    (2, 48, 1536, 128, 1),                     # 8-wave blocks, 8 | B*H, several rounds
    (4, 30, 777, 96, 0),
])
def test_grids_larger_than_the_chip(B, H, N, d, mask):
    """Grids with more work items than resident workgroups (each workgroup
    loops over several items), with head counts that do and do not divide
    by the XCD count, ragged N and mixed key lengths, on every element."""
    kv_range = (1, N) if mask & MASK_KEY_PADDING else None
    x = make_raw(B, H, N, d, "bf16", seed=B * 1000 + H + N + d, q_mult=2.0,
                 kv_len_range=kv_range)
    scale = d ** -0.5
    what = f"fa_fwd B={B} H={H} N={N} d={d} mask={mask}"
    say(what)
    O, L = _run(x, scale, mask, -1, "bhnd", True)
    ref = attention_general_ref(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]), scale, mask, -1,
                                x.get("kv_lens"), magnitudes=True)
    compare_bound(O, L, ref, what)


@pytest.mark.parametrize("d,mask", [(64, MASK_KEY_PADDING), (128, MASK_KEY_PADDING | 1)])
def test_looping_workgroups_with_empty_and_edge_key_lengths(d, mask):
    """Items without any visible key (kv_len = 0) and key lengths at block
    edges inside a grid larger than the chip: looping workgroups must skip
    the empty items' key loop, write O = 0 and LSE = -inf for them, and keep
    their LDS buffers consistent for the next item."""
    B, H, N = 9, 32, 600
    x = make_raw(B, H, N, d, "bf16", seed=4242 + d, q_mult=2.0, kv_len_range=(1, N))
    x["kv_lens"] = np.array([0, 1, 64, 128, 0, N, 129, 0, 383], dtype=np.int32)
    scale = d ** -0.5
    what = f"fa_fwd B={B} H={H} N={N} d={d} mask={mask} kv={x['kv_lens'].tolist()}"
    say(what)
    O, L = _run(x, scale, mask, -1, "bhnd", True)
    ref = attention_general_ref(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]), scale, mask, -1,
                                x["kv_lens"], magnitudes=True)
    compare_bound(O, L, ref, what)
