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
