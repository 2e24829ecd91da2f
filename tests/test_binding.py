"""The Python binding refuses tensors the kernels cannot take (host memory,
wrong dtype, wrong shape) before it reaches the library: a stub stands in for
libfa92.so and fails the test if any entry point is called."""
import pytest
import torch

import exact_attention_92_amd as fa


class _NoCalls:
    def __getattr__(self, name):
        raise AssertionError(f"{name} was reached with arguments the binding must refuse")


@pytest.fixture(autouse=True)
def stub_library(monkeypatch):
    monkeypatch.setattr(fa, "_lib", _NoCalls())


def _bhnd(dtype=torch.bfloat16, B=2, H=3, N=70, d=64):
    return torch.zeros((B, H, N, d), dtype=dtype)


def _calls(dtype=torch.bfloat16):
    """One call of every entry point with well-shaped tensors in host memory."""
    q = _bhnd(dtype)
    lse = torch.zeros((2, 3, 70))
    kv = torch.full((2,), 70, dtype=torch.int32)
    u8 = _bhnd(torch.uint8)
    ds = torch.ones((2, 3))
    qp, pool = torch.zeros((2, 3, 64), dtype=dtype), torch.zeros((8, 3, 16, 64), dtype=dtype)
    tables, lens = torch.zeros((2, 4), dtype=torch.int32), torch.full((2,), 5, dtype=torch.int32)
    packed = torch.zeros((100, 3, 64), dtype=dtype)
    cu = torch.tensor([0, 40, 100], dtype=torch.int32)
    return {
        "fa_fwd": lambda: fa.fa_fwd(q, q, q, q.clone(), lse, 0.1, 2, kv),
        "fa_fwd_f32": lambda: fa.fa_fwd_f32(q.float(), q.float(), q.float(), q.float(), lse,
                                            0.1),
        "fa_fwd_general": lambda: fa.fa_fwd_general(q, q, q, q.clone(), lse, 0.1, 2, 5, kv),
        "fa_fwd_varlen": lambda: fa.fa_fwd_varlen(packed, packed, packed, packed.clone(),
                                                  torch.zeros((3, 100)), cu, cu, 60, 0.1),
        "fa_fwd_fp8": lambda: fa.fa_fwd_fp8(u8, u8, u8, ds, ds, ds, q.clone(), lse, 0.1),
        "fa_bwd": lambda: fa.fa_bwd(q, q, q, q, lse, q, q.clone(), q.clone(), q.clone(),
                                    lse.clone(), 0.1),
        "fa_decode_paged": lambda: fa.fa_decode_paged(qp, pool, pool, tables, lens,
                                                      qp.clone(), torch.zeros((2, 3)),
                                                      torch.zeros(1 << 16), 0.1),
    }


@pytest.mark.parametrize("name", sorted(_calls()))
def test_host_tensors_are_refused(name):
    with pytest.raises(ValueError, match="device memory"):
        _calls()[name]()


@pytest.mark.parametrize("name", ["fa_fwd", "fa_fwd_general", "fa_fwd_varlen", "fa_bwd",
                                  "fa_decode_paged"])
def test_wrong_dtype_is_refused(name):
    with pytest.raises(TypeError):
        _calls(torch.float16)[name]()


def test_check_names_the_problem():
    with pytest.raises(TypeError, match="lse"):
        fa._check("lse", torch.zeros(3, dtype=torch.float64), torch.float32)
    with pytest.raises(TypeError, match="kv_lens"):
        fa._check("kv_lens", [1, 2], torch.int32)


def test_overlapping_view_detection():
    """The stride rule that keeps overlapping output views away from the
    general forward: dense and permuted layouts pass, expanded or aliasing
    views do not, strided views with gaps pass."""
    x = torch.empty(2, 3, 10, 8)
    assert not fa._overlapping(x)
    assert not fa._overlapping(x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3))
    assert not fa._overlapping(x[:, :, ::2])
    assert not fa._overlapping(torch.empty(1, 3, 10, 8))
    assert fa._overlapping(torch.empty(1, 3, 10, 8).expand(2, 3, 10, 8))
    assert fa._overlapping(torch.empty(2, 10, 8).unsqueeze(1).expand(2, 3, 10, 8))
    assert fa._overlapping(torch.empty(2, 3, 80).as_strided((2, 3, 10, 8), (240, 80, 4, 1)))
