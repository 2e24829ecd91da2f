"""On the GPU: the binding refuses a single bad tensor among good device
tensors (host memory, a strided or expanded view where a dense buffer is
needed) and nothing is written."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")
    import exact_attention_92_amd as fa
    fa.load_library()


def _nan(shape, dtype):
    import torch
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def test_one_bad_tensor_is_refused_and_nothing_is_written():
    import torch

    import exact_attention_92_amd as fa
    B, H, N, d = 2, 3, 70, 64
    q = torch.randn((B, H, N, d), device="cuda").to(torch.bfloat16)
    o = _nan((B, H, N, d), torch.bfloat16)
    lse = _nan((B, H, N), torch.float32)
    kv = torch.full((B,), N, dtype=torch.int32, device="cuda")
    kv_strided = torch.full((2 * B,), N, dtype=torch.int32, device="cuda")[::2]
    cases = {
        "fa_fwd host lse": lambda: fa.fa_fwd(q, q, q, o, lse.cpu(), 0.1),
        "fa_fwd strided kv_lens": lambda: fa.fa_fwd(q, q, q, o, lse, 0.1, 2, kv_strided),
        "fa_fwd_general host lse": lambda: fa.fa_fwd_general(q, q, q, o, lse.cpu(), 0.1),
        "fa_fwd_general host kv_lens": lambda: fa.fa_fwd_general(q, q, q, o, lse, 0.1, 2, -1,
                                                                 kv.cpu()),
        "fa_fwd_general overlapping o": lambda: fa.fa_fwd_general(
            q, q, q, _nan((1, H, N, d), torch.bfloat16).expand(B, H, N, d), lse, 0.1),
        "fa_fwd_general o rows aliasing heads": lambda: fa.fa_fwd_general(
            q, q, q, _nan((B, N, d), torch.bfloat16).unsqueeze(1).expand(B, H, N, d), lse, 0.1),
        "fa_bwd strided dq": lambda: fa.fa_bwd(
            q, q, q, q, lse, q, _nan((B, H, N, 2 * d), torch.bfloat16)[..., ::2],
            o, o.clone(), lse.clone(), 0.1),
    }
    packed = torch.randn((100, H, d), device="cuda").to(torch.bfloat16)
    po = _nan((100, H, d), torch.bfloat16)
    cu = torch.tensor([0, 40, 100], dtype=torch.int32, device="cuda")
    cases["fa_fwd_varlen host lse"] = lambda: fa.fa_fwd_varlen(
        packed, packed, packed, po, torch.zeros((H, 100)), cu, cu, 60, 0.1)
    qd = torch.randn((B, H, d), device="cuda").to(torch.bfloat16)
    pool = torch.randn((8, H, 16, d), device="cuda").to(torch.bfloat16)
    tables = torch.zeros((B, 4), dtype=torch.int32, device="cuda")
    lens = torch.full((B,), 5, dtype=torch.int32, device="cuda")
    od, lsed = _nan((B, H, d), torch.bfloat16), _nan((B, H), torch.float32)
    need = fa.fa_decode_paged_workspace_bytes(B, H, d, 16, 4)
    ws = torch.zeros(1, device="cuda").expand(need // 4 + 1)
    cases["fa_decode_paged expanded workspace"] = lambda: fa.fa_decode_paged(
        qd, pool, pool, tables, lens, od, lsed, ws, 0.1)
    for what, call in cases.items():
        with pytest.raises(ValueError):
            call()
    torch.cuda.synchronize()
    for t in (o, lse, po, od, lsed):
        assert torch.isnan(t.float()).all()
