"""The Python binding's argument checks, on the CPU.

The kernels take raw device pointers, so the binding checks, before the
library is called, every tensor's dtype, exact shape and contiguity and that
it lives on the GPU holding q (a host tensor's address handed to a kernel
would make it read or write memory that is not the tensor's).  Here the
library entry points are replaced by functions that fail the test, so each
case shows that its check raises before any library call.
"""
import pytest
import torch

from io_aware_attention_fwd_amd import _lib


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def forbidden(*a, **k):
        raise AssertionError("the library was called although an argument check should have raised")

    for name in ("load", "fa_fwd", "fa_fwd_fp8", "fa_fwd_varlen", "fa_fwd_dropout", "fa_bwd", "fa_qkv_proj"):
        monkeypatch.setattr(_lib, name, forbidden)


def _t(*shape, dtype=torch.float16):
    return torch.zeros(*shape, dtype=dtype)


B, H, N, d = 2, 3, 40, 64


def test_fwd_host_tensors_rejected():
    q = _t(B, H, N, d)
    with pytest.raises(ValueError, match="on a GPU"):
        _lib.fwd(q, q.clone(), q.clone(), 0.1)


@pytest.mark.parametrize("out_shape", [(B, H, N, d + 1), (B * H * N * d,), (B, H, N - 1, d)])
def test_fwd_out_wrong_shape(out_shape):
    q = _t(B, H, N, d)
    with pytest.raises(ValueError, match="out must have shape"):
        _lib.fwd(q, q, q, 0.1, out=_t(*out_shape))


def test_fwd_out_non_contiguous():
    q = _t(B, H, N, d)
    out = _t(B, H, d, N).transpose(2, 3)
    with pytest.raises(ValueError, match="out must be contiguous"):
        _lib.fwd(q, q, q, 0.1, out=out)


def test_fwd_out_wrong_dtype():
    q = _t(B, H, N, d)
    with pytest.raises(TypeError, match="out must be"):
        _lib.fwd(q, q, q, 0.1, out=_t(B, H, N, d, dtype=torch.bfloat16))


@pytest.mark.parametrize("lse", [_t(B, H, N + 1, dtype=torch.float32), _t(B, H, N, dtype=torch.float16),
                                 _t(B, N, H, dtype=torch.float32).transpose(1, 2)])
def test_fwd_lse_rejected(lse):
    q = _t(B, H, N, d)
    with pytest.raises((ValueError, TypeError), match="lse must"):
        _lib.fwd(q, q, q, 0.1, lse=lse)


def test_fwd_fp8_out_must_be_bf16():
    q = torch.zeros(B, H, N, d, dtype=torch.uint8)
    with pytest.raises(TypeError, match="out must be"):
        _lib.fwd(q, q, q, 0.1, out=_t(B, H, N, d))


def test_varlen_checks():
    q = _t(50, H, d)
    cu = torch.tensor([0, 20, 50], dtype=torch.int32)
    with pytest.raises(ValueError, match="on a GPU"):
        _lib.fwd_varlen(q, q, q, cu, 30, 0.1)
    with pytest.raises(ValueError, match="out must have shape"):
        _lib.fwd_varlen(q, q, q, cu, 30, 0.1, out=_t(50, H, d + 64))
    with pytest.raises(ValueError, match="lse must have shape"):
        _lib.fwd_varlen(q, q, q, cu, 30, 0.1, lse=_t(50, H, dtype=torch.float32))
    with pytest.raises(TypeError, match="cu_seqlens"):
        _lib.fwd_varlen(q, q, q, cu.long(), 30, 0.1)


def test_dropout_host_tensors_rejected():
    q = _t(B, H, N, d)
    with pytest.raises(ValueError, match="on a GPU"):
        _lib.fwd_dropout(q, q, q, 0.1, False, 0.1, 7)


def test_bwd_checks():
    q = _t(B, H, N, d)
    lse = _t(B, H, N, dtype=torch.float32)
    with pytest.raises(ValueError, match="on a GPU"):
        _lib.bwd(q, q, q, q, lse, q, 0.1)
    with pytest.raises(ValueError, match="lse"):
        _lib.bwd(q, q, q, q, lse[:, :, :-1], q, 0.1)
    with pytest.raises(ValueError):
        _lib.bwd(q, q, q, _t(B, H, N, d + 1), lse, q, 0.1)


def test_proj_checks():
    x = _t(2, 10, 128)
    w = _t(3 * H * d, 128)
    with pytest.raises(ValueError, match="on a GPU"):
        _lib.qkv_proj(x, w, None, H, d)
    with pytest.raises(ValueError):
        _lib.qkv_proj(x, _t(3 * H * d + 1, 128), None, H, d)


def test_same_device_helper_names_the_offender():
    """A tensor on another device than q is named in the error (checked with a
    stand-in 'GPU' device, since this machine has none)."""

    class Dev:
        def __init__(self, t, dev):
            self.device = torch.device(dev)

    ref = Dev(None, "cuda:0")
    with pytest.raises(ValueError, match="k is on cpu"):
        _lib._same_device(ref, None, k=Dev(None, "cpu"))
    with pytest.raises(ValueError, match="lse is on cuda:1"):
        _lib._same_device(ref, None, k=Dev(None, "cuda:0"), lse=Dev(None, "cuda:1"))
    _lib._same_device(ref, None, k=Dev(None, "cuda:0"), bias=None)
