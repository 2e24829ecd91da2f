"""The no-allocation decode entry point (fa_decode_paged_noalloc), called
through the C ABI: its output must equal fa_decode_paged's on the same inputs
(the same kernels, with the library's fixed per-GPU buffer as their scratch
instead of a caller workspace), bit for bit, on two calls in a row -- the
second smaller, so stale partial results from the first must not leak in --
and sizes past the buffer must be refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest

from fa_inputs import make_paged_decode
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")
    import exact_attention_92_amd as fa
    return fa.load_library()


def _upload(x):
    import torch

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return (bf(x["q"]), bf(x["k_pool"]), bf(x["v_pool"]),
            torch.from_numpy(x["block_tables"]).cuda(), torch.from_numpy(x["seq_lens"]).cuda())


def _both(lib, x, scale):
    """(O, LSE) of fa_decode_paged and of fa_decode_paged_noalloc, both called
    through the C ABI on the default stream."""
    import torch
    q, kp, vp, tab, lens = _upload(x)
    B, H, d = q.shape
    nblk, _, bs, _ = kp.shape
    vptr = ctypes.c_void_p
    out = []
    for noalloc in (False, True):
        o = torch.full((B, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, H), float("nan"), device="cuda")
        args = [vptr(t.data_ptr()) for t in (q, kp, vp, tab, lens, o, lse)]
        if noalloc:
            st = lib.fa_decode_paged_noalloc(*args, B, H, d, bs, tab.shape[1], nblk,
                                             ctypes.c_float(scale), None)
        else:
            need = lib.fa_decode_paged_workspace_bytes(B, H, d, bs, tab.shape[1])
            ws = torch.full(((need + 3) // 4,), float("nan"), device="cuda")
            st = lib.fa_decode_paged(*args, vptr(ws.data_ptr()), B, H, d, bs, tab.shape[1],
                                     nblk, ctypes.c_float(scale), None)
        assert st == 0, st
        torch.cuda.synchronize()
        out.append((o.view(torch.int16).cpu().numpy(), lse.cpu().numpy()))
    return out


def test_noalloc_matches_workspace_entry_point_twice(lib):
    # First call: 24 requests x 8 heads, up to 3000 tokens (6 chunks of
    # partial results each); second: 5 requests x 4 heads, up to 700 tokens,
    # one of them empty, so most of the buffer still holds the first call's
    # partial results.
    cases = [(dict(B=24, H=8, d=128, block_size=64, len_range=(1, 3000), seed=71), 0.088),
             (dict(B=5, H=4, d=64, block_size=16, len_range=(0, 700), seed=72,
                   lens=[0, 585, 1, 300, 700]), 0.125)]
    for kw, scale in cases:
        x = make_paged_decode(kw["B"], kw["H"], kw["d"], kw["block_size"], kw["len_range"],
                              kw["seed"], lens=kw.get("lens"))
        say(f"  noalloc decode B={kw['B']} H={kw['H']} d={kw['d']} bs={kw['block_size']} "
            f"lens={x['seq_lens'].min()}..{x['seq_lens'].max()}")
        (o_ws, l_ws), (o_na, l_na) = _both(lib, x, scale)
        assert not np.isnan(l_ws).any()
        assert np.array_equal(o_na, o_ws), "O differs from fa_decode_paged"
        assert np.array_equal(l_na.view(np.uint32), l_ws.view(np.uint32)), "LSE differs"


def test_noalloc_refuses_sizes_past_its_buffer(lib):
    import torch

    import exact_attention_92_amd as fa
    # 64 x 32 x 128 with 8192-token tables needs 17.0 MB of partial results.
    B, H, d, bs, mb = 64, 32, 128, 64, 128
    need = lib.fa_decode_paged_workspace_bytes(B, H, d, bs, mb)
    assert need > fa.DECODE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, d), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((4, H, bs, d), dtype=torch.bfloat16, device="cuda")
    tab = torch.zeros((B, mb), dtype=torch.int32, device="cuda")
    lens = torch.zeros((B,), dtype=torch.int32, device="cuda")
    o = torch.full((B, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H), float("nan"), device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fa_decode_paged_noalloc(q, pool, pool, tab, lens, o, lse, 0.1)
    assert e.value.status == fa.FA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all() and torch.isnan(lse).all()     # nothing enqueued
