"""The Python binding rejects tensors that do not match the problem before any call
into libmoda (CPU only).  The C ABI takes bare pointers, so a transposed view, a
layer-major depth tensor, a short depth tensor or a wrong dtype could otherwise
give wrong results or reads past an allocation."""
import pytest
import torch

from transformer_attention_moda_amd import binding as mb

B, Hq, Hk, T, d, L = 1, 4, 2, 16, 64, 3
BF = torch.bfloat16


def tensors(dtype=BF):
    z = lambda *s: torch.zeros(s, dtype=dtype)  # noqa: E731
    return dict(Q=z(B, Hq, T, d), K=z(B, Hk, T, d), V=z(B, Hk, T, d), Kd=z(B, Hk, T * L, d),
                Vd=z(B, Hk, T * L, d), O=z(B, Hq, T, d), lse=torch.zeros(B, Hq, T),
                dO=z(B, Hq, T, d), dQ=z(B, Hq, T, d), dK=z(B, Hk, T, d), dV=z(B, Hk, T, d),
                dKd=z(B, Hk, T * L, d), dVd=z(B, Hk, T * L, d))


def call_fwd(x, p=None):
    p = p or mb.problem(B, Hq, Hk, T, d, L)
    mb.moda_fwd(p, x["Q"], x["K"], x["V"], x["Kd"], x["Vd"], x["O"], x["lse"])


def call_bwd(x, ws=None):
    p = mb.problem(B, Hq, Hk, T, d, L)
    mb.moda_bwd(p, x["Q"], x["K"], x["V"], x["Kd"], x["Vd"], x["O"], x["lse"], x["dO"],
                x["dQ"], x["dK"], x["dV"], x["dKd"], x["dVd"],
                ws if ws is not None else torch.zeros(4096, dtype=torch.uint8))


@pytest.fixture(autouse=True)
def no_library_calls(monkeypatch):
    """Any call that reaches the C library fails the test: validation must raise first."""
    def boom(*a, **k):
        raise AssertionError("reached libmoda")
    monkeypatch.setattr(mb, "load", boom)


def test_host_tensors_are_rejected():
    with pytest.raises(ValueError, match="not on a GPU"):
        call_fwd(tensors())


def test_transposed_view_is_rejected():
    x = tensors()
    x["Q"] = torch.zeros(B, T, Hq, d, dtype=BF).transpose(1, 2)   # right shape, wrong strides
    with pytest.raises(ValueError, match="not contiguous"):
        call_fwd(x)


def test_layer_major_depth_tensor_is_rejected():
    x = tensors()
    x["Kd"] = torch.zeros(L, B, Hk, T, d, dtype=BF)     # same element count, natural layout
    with pytest.raises(ValueError, match="shape"):
        call_fwd(x)


def test_short_depth_tensor_is_rejected():
    x = tensors()
    x["Vd"] = torch.zeros(B, Hk, T * L - 1, d, dtype=BF)
    with pytest.raises(ValueError, match="shape"):
        call_fwd(x)


@pytest.mark.parametrize("name", ["K", "V", "Kd", "O"])
def test_mixed_dtypes_are_rejected(name):
    x = tensors()
    x[name] = x[name].float()
    with pytest.raises(TypeError, match=name):
        call_fwd(x)


def test_lse_must_be_fp32():
    x = tensors()
    x["lse"] = x["lse"].to(BF)
    with pytest.raises(TypeError, match="lse"):
        call_fwd(x)


def test_missing_depth_only_allowed_without_depth():
    x = tensors()
    x["Kd"] = None
    with pytest.raises(ValueError, match="Kd is required"):
        call_fwd(x)
    x0 = tensors()
    x0["Kd"] = x0["Vd"] = None
    with pytest.raises(ValueError, match="not on a GPU"):      # L = 0: depth may be absent
        call_fwd(x0, mb.problem(B, Hq, Hk, T, d, 0))


@pytest.mark.parametrize("name", ["dO", "dQ", "dK", "dV", "dKd", "dVd"])
def test_backward_gradient_shapes_are_checked(name):
    x = tensors()
    x[name] = x[name][..., :-1].contiguous()
    with pytest.raises(ValueError, match=name):
        call_bwd(x)


def test_pack_depth_shapes_are_checked():
    p = mb.problem(B, Hk, Hk, T, d, L, 1.0)
    with pytest.raises(ValueError, match="layers"):
        mb.moda_pack_depth(p, torch.zeros(B, Hk, T * L, d, dtype=BF),
                           torch.zeros(B, Hk, T * L, d, dtype=BF))
    with pytest.raises(ValueError, match="layers"):
        mb.pack_depth(torch.zeros(B, Hk, T, d, dtype=BF))


def test_depth_kv_cache_shapes_and_host_append():
    """DepthKVCache holds the packed [B,Hk,T*L,d] pair; empty sizes are refused, and an append
    into host tensors is refused before any launch."""
    with pytest.raises(ValueError):
        mb.DepthKVCache(B, Hk, T, 0, d, device="cpu")
    c = mb.DepthKVCache(B, Hk, T, L, d, device="cpu")
    Kd, Vd = c.tensors()
    assert Kd.shape == (B, Hk, T * L, d) and Vd.shape == Kd.shape and Kd.dtype == BF
    layer = torch.zeros(B, Hk, T, d, dtype=BF)
    with pytest.raises(ValueError, match="GPU"):
        c.append(layer, layer, 0)
