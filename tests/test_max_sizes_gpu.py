"""The largest sequence lengths the forward entry points accept, on the GPU.

Each entry point addresses one head's rows with 32-bit byte offsets and so
bounds N (the limits are stated in include/fa_api.h).  These tests run at
exactly that bound, with masks that keep the work small (key padding to a
few hundred keys, or a causal 64-key window, so every key row is read), and
check sampled query rows -- the first, around the 2^31-byte mark, and the
last blocks -- against the oracle element by element, every output for being
written, and that one row more is refused.  The inputs are drawn on the
device from seeded generators (drawing them on the host would take tens of
GB); only the sampled rows and the keys they see are copied back.
"""
import numpy as np
import pytest

from fa_inputs import MASK_CAUSAL, MASK_KEY_PADDING, MASK_NONE
from gpu_util import compare, compare_bound, say
from oracle import attention_general_ref

pytestmark = pytest.mark.gpu
KV = 200          # visible keys with key padding
WINDOW = 64       # keys before a query's own position with a window
LIMIT = 2 ** 32 - 1


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")
    import exact_attention_92_amd as fa
    fa.load_library()
    yield
    torch.cuda.empty_cache()


def _rows(N, row_bytes):
    mid = 2 ** 31 // row_bytes           # the row that starts at byte 2^31 (if any)
    r = {0, 1, 63, 64, 255, 256, mid - 1, mid, mid + 1, N // 2, N - 257, N - 256, N - 129,
         N - 65, N - 64, N - 2, N - 1}
    return np.array(sorted(x for x in r if 0 <= x < N))


def _draw(shape, dtype, seed):
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=dtype)


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _at(t, rows):
    """Rows ``rows`` (numpy indices) of a [1, 1, N, ...] device tensor."""
    import torch
    return t[:, :, torch.as_tensor(rows, device=t.device)]


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def _key_padding_case(dtype, d, N, entry):
    import torch

    import exact_attention_92_amd as fa
    q, k, v = (_draw((1, 1, N, d), dtype, s) for s in (11, 12, 13))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, 1, N), float("nan"), device="cuda")
    kv = torch.tensor([KV], dtype=torch.int32, device="cuda")
    scale = d ** -0.5
    getattr(fa, entry)(q, k, v, o, lse, scale, MASK_KEY_PADDING, kv)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any().item() and torch.isfinite(lse).all().item()
    rows = _rows(N, d * q.element_size())
    Or, Lr, M = attention_general_ref(_f64(q[:, :, rows]), _f64(k[:, :, :KV]),
                                      _f64(v[:, :, :KV]), scale, MASK_NONE, -1, None,
                                      magnitudes=True)
    O, L = _f64(o[:, :, rows]), _f64(lse[:, :, rows])
    # One row more is refused before anything is enqueued (the pointers are
    # not read: the size check comes first).
    st = getattr(fa.load_library(), entry)(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                           o.data_ptr(), lse.data_ptr(), 1, 1, N + 1, d,
                                           scale, MASK_KEY_PADDING, kv.data_ptr(), _stream())
    assert st == fa.FA_ERR_INVALID_ARG
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return O, L, (Or, Lr, M)


def test_fa_fwd_bf16_largest_n():
    import torch
    d = 64
    N = LIMIT // (d * 4) - 256                  # (N + 256) d 4 <= 2^32 - 1
    assert (N + 257) * d * 4 > LIMIT
    what = f"fa_fwd bf16 B=1 H=1 N={N} d={d} key padding {KV}"
    say(what)
    O, L, ref = _key_padding_case(torch.bfloat16, d, N, "fa_fwd")
    compare_bound(O, L, ref, what)


def test_fa_fwd_f32_largest_n():
    import torch
    d = 64
    N = LIMIT // (d * 4) - 128                  # (N + 128) d 4 <= 2^32 - 1
    assert (N + 129) * d * 4 > LIMIT
    what = f"fa_fwd_f32 B=1 H=1 N={N} d={d} key padding {KV}"
    say(what)
    O, L, (Or, Lr, _) = _key_padding_case(torch.float32, d, N, "fa_fwd_f32")
    compare(O, L, Or, Lr, "f32", what)


def test_fa_fwd_general_largest_n_windowed():
    """Causal with a 64-key window: every key row up to the end is read."""
    import torch

    import exact_attention_92_amd as fa
    d = 128
    N = LIMIT // (d * 2) - 256                  # (rows + 256) row_stride 2 <= 2^32 - 1
    assert (N + 257) * d * 2 > LIMIT
    what = f"fa_fwd_general B=1 H=1 Nq=Nk={N} d={d} causal window {WINDOW}"
    say(what)
    q, k, v = (_draw((1, 1, N, d), torch.bfloat16, s) for s in (21, 22, 23))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, 1, N), float("nan"), device="cuda")
    scale = d ** -0.5
    fa.fa_fwd_general(q, k, v, o, lse, scale, MASK_CAUSAL, WINDOW)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any().item() and torch.isfinite(lse).all().item()
    rows = _rows(N, d * 2)
    refs = []
    for r in rows:
        lo = max(0, int(r) - WINDOW)
        refs.append(attention_general_ref(_f64(q[:, :, r:r + 1]), _f64(k[:, :, lo:r + 1]),
                                          _f64(v[:, :, lo:r + 1]), scale, MASK_CAUSAL, WINDOW,
                                          None, magnitudes=True))
    ref = tuple(np.concatenate([x[i] for x in refs], axis=2) for i in range(3))
    O, L = _f64(o[:, :, rows]), _f64(lse[:, :, rows])
    lib = fa.load_library()
    st = lib.fa_fwd_general(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                            lse.data_ptr(), 1, 1, N + 1, N + 1, d, None, None, None, None, scale,
                            MASK_CAUSAL, WINDOW, None, _stream())
    assert st == fa.FA_ERR_INVALID_ARG
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    compare_bound(O, L, ref, what)


def test_fa_bwd_largest_n():
    """The backward at its bound ((N + 256) d 4 <= 2^32 - 1) with key padding
    to 200 keys.  dQ and the row sums on sampled rows against the oracle
    (the sampled rows placed first in a 200-row query block: unmasked rows
    are independent); keys no row sees have dK = dV = 0 exactly; over the
    visible keys every row's dS sums to 0 and P to 1, so sum_c dK_c = 0 and
    sum_c dV_c = sum_r dO_r."""
    import torch

    import exact_attention_92_amd as fa
    from gpu_util import compare_grads
    from oracle import attention_bwd_ref
    d = 64
    N = LIMIT // (d * 4) - 256
    what = f"fa_bwd B=1 H=1 N={N} d={d} key padding {KV}"
    say(what)
    q, k, v, do = (_draw((1, 1, N, d), torch.bfloat16, s) for s in (31, 32, 33, 34))
    kv = torch.tensor([KV], dtype=torch.int32, device="cuda")
    scale = d ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, N), device="cuda")
    fa.fa_fwd(q, k, v, o, lse, scale, MASK_KEY_PADDING, kv)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    dps = torch.full((1, 1, N), float("nan"), device="cuda")
    fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, dps, scale, MASK_KEY_PADDING, kv)
    torch.cuda.synchronize()
    for t in (dq, dk, dv, dps):
        assert not torch.isnan(t).any().item()
    assert (dk[:, :, KV:] == 0).all().item() and (dv[:, :, KV:] == 0).all().item()
    dv_sum = dv[:, :, :KV].double().sum(dim=2)
    do_sum = do.double().sum(dim=2)
    assert (dv_sum - do_sum).abs().max().item() <= 2e-2 * N ** 0.5, "sum dV"
    dk_vis = dk[:, :, :KV].double()
    assert (dk_vis.sum(dim=2).abs() <= 1e-2 * dk_vis.abs().sum(dim=2)).all().item(), "sum dK"
    rows = _rows(N, d * 2)
    R = len(rows)
    qs, dos = np.zeros((1, 1, KV, d)), np.zeros((1, 1, KV, d))
    qs[:, :, :R], dos[:, :, :R] = _f64(_at(q, rows)), _f64(_at(do, rows))
    dQ, _, _, DP, M = attention_bwd_ref(qs, _f64(k[:, :, :KV]), _f64(v[:, :, :KV]), dos, scale,
                                        MASK_NONE, rows=np.arange(R), magnitudes=True)
    g = {"dq": _f64(_at(dq, rows)), "dps": _f64(_at(dps, rows))}
    ref = {"dq": dQ[:, :, :R], "dps": DP[:, :, :R]}
    mag = {"dq": M["dq"][:, :, :R], "dps": M["dps"][:, :, :R]}
    st = fa.load_library().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                  dv.data_ptr(), dps.data_ptr(), 1, 1, N + 1, d, scale,
                                  MASK_KEY_PADDING, kv.data_ptr(), _stream())
    assert st == fa.FA_ERR_INVALID_ARG
    del q, k, v, do, o, lse, dq, dk, dv, dps
    torch.cuda.empty_cache()
    compare_grads(g, ref, mag, what, keys=("dq", "dps"))


def test_fa_fwd_varlen_largest_total():
    """Packed sequences filling the bound ((total + 256) H d 2 <= 2^32 - 1):
    a short sequence, one of nearly all the rows, and another short one,
    causal with a 64-key window; sampled rows of each sequence (its first and
    last rows, and around byte 2^31 of the packed tensors) against the
    oracle over the keys each row sees."""
    import torch

    import exact_attention_92_amd as fa
    H, d, W = 1, 64, WINDOW
    total = LIMIT // (H * d * 2) - 256
    assert (total + 257) * H * d * 2 > LIMIT
    lens = [300, total - 600, 300]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    what = f"fa_fwd_varlen H={H} d={d} lengths={lens} causal window {W}"
    say(what)
    q, k, v = (_draw((total, H, d), torch.bfloat16, s) for s in (41, 42, 43))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((H, total), float("nan"), device="cuda")
    cu_d = torch.from_numpy(cu).cuda()
    scale = d ** -0.5
    fa.fa_fwd_varlen(q, k, v, o, lse, cu_d, cu_d, max(lens), scale, MASK_CAUSAL, W)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any().item() and torch.isfinite(lse).all().item()
    mid = 2 ** 31 // (H * d * 2)
    picks = []
    for s0, s1 in zip(cu[:-1], cu[1:]):
        picks += [s0, s0 + 1, s0 + 64, s1 - 65, s1 - 2, s1 - 1]
    picks += [mid - 1, mid, mid + 1]
    rows = np.array(sorted(set(int(x) for x in picks)))
    Os, Ls, refs = [], [], []
    for g_row in rows:
        s = int(np.searchsorted(cu, g_row, side="right") - 1)
        lo = max(int(cu[s]), int(g_row) - W)
        sl = lambda t, a, b: _f64(t[a:b].permute(1, 0, 2))[None]     # [1, H, rows, d]
        refs.append(attention_general_ref(sl(q, g_row, g_row + 1), sl(k, lo, g_row + 1),
                                          sl(v, lo, g_row + 1), scale, MASK_CAUSAL, W, None,
                                          magnitudes=True))
        Os.append(sl(o, g_row, g_row + 1))
        Ls.append(_f64(lse[:, g_row:g_row + 1])[None])
    ref = tuple(np.concatenate([x[i] for x in refs], axis=2) for i in range(3))
    O, L = np.concatenate(Os, axis=2), np.concatenate(Ls, axis=2)
    st = fa.load_library().fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                         lse.data_ptr(), cu_d.data_ptr(), cu_d.data_ptr(), 3, H,
                                         d, total + 1, total, max(lens), scale, MASK_CAUSAL, W,
                                         _stream())
    assert st == fa.FA_ERR_INVALID_ARG
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    compare_bound(O, L, ref, what)
