"""GPU parity of the fused QKV projection ``fa_qkv_proj`` against the oracle.

Bar per element: |y_gpu - y_ref| <= ulp(y_ref) + 2^-20 * sum_k |x_k w_k|.
The kernel accumulates the D products in float32 and rounds once to the
16-bit output: the accumulation error stays far below 2^-20 of the sum of
absolute products (D <= 4096 terms of relative error 2^-24), and the final
rounding moves the value by half an ulp, or one ulp where the accumulation
error lands it on the other side of a rounding boundary.  ulp is that of the
output format at |y_ref| (2^-10 relative for binary16, 2^-7 for bfloat16).

End to end, the projection feeds ``fa_fwd``; the oracle attention runs on the
oracle's projection rounded to the same storage format, within the forward
pass's bar.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from io_aware_attention_fwd_amd import _lib, gen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}
_MANT = {"f16": 10, "bf16": 7}
_MIN_EXP = {"f16": -14, "bf16": -126}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()


def _dev(a, dtype):
    if dtype == "f16":
        return torch.from_numpy(a).cuda()
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def _host(a, dtype):
    return oracle.dequantize(a, dtype, 1.0)


def _ulp(y, dtype):
    e = np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** _MIN_EXP[dtype])))
    return 2.0 ** (e - _MANT[dtype])


def _run(pi: gen.ProjectionInputs, use_bias=True):
    x, w = _dev(pi.x, pi.dtype), _dev(pi.w, pi.dtype)
    b = _dev(pi.bias, pi.dtype) if use_bias else None
    q, k, v = _lib.qkv_proj(x, w, b, pi.H, pi.d)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy().astype(np.float64) for t in (q, k, v)]


def _check(pi: gen.ProjectionInputs, outs, use_bias=True):
    x, w = _host(pi.x, pi.dtype), _host(pi.w, pi.dtype)
    bias = _host(pi.bias, pi.dtype) if use_bias else None
    refs = oracle.qkv_projection(x, w, bias, pi.H, pi.d)
    absum = oracle.qkv_projection(np.abs(x), np.abs(w), None, pi.H, pi.d)
    worst = 0.0
    for s, (got, ref, a) in enumerate(zip(outs, refs, absum)):
        bound = _ulp(ref, pi.dtype) + 2.0 ** -20 * a
        ratio = (np.abs(got - ref) / bound).max()
        assert ratio <= 1.0, f"tensor {'QKV'[s]}: error {ratio:.3g} x the bar"
        worst = max(worst, ratio)
    return worst


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("B,N,D,H,d", [
    (2, 100, 64, 2, 64),     # one k step, ragged token tile, 3 feature tiles
    (1, 300, 512, 3, 128),   # several k steps, 9 feature tiles
    (3, 257, 1024, 5, 64),   # feature count 960: a partial feature tile
])
def test_projection_parity(dtype, B, N, D, H, d):
    print(f"[proj] B={B} N={N} D={D} H={H} d={d} {dtype}", flush=True)
    pi = gen.make_projection(B, N, D, H, d, dtype, seed=1)
    worst = _check(pi, _run(pi))
    print(f"[proj] worst error / bar {worst:.3g}")


def test_projection_without_bias():
    pi = gen.make_projection(2, 130, 256, 2, 64, "bf16", seed=2)
    outs = _run(pi, use_bias=False)
    _check(pi, outs, use_bias=False)
    zero = gen.ProjectionInputs(pi.dtype, pi.x, pi.w, np.zeros_like(pi.bias), pi.H, pi.d)
    for a, b in zip(outs, _run(zero)):
        assert np.array_equal(a, b)  # a zero bias and no bias give the same bits


def test_projection_full_size():
    B, N, D, H, d, dtype = 4, 1024, 2048, 32, 64, "f16"
    print(f"[proj] full size B={B} N={N} D={D} H={H} d={d} {dtype}", flush=True)
    pi = gen.make_projection(B, N, D, H, d, dtype, seed=3)
    worst = _check(pi, _run(pi))
    print(f"[proj] worst error / bar {worst:.3g}")


@pytest.mark.parametrize("dtype,causal", [("f16", False), ("bf16", True)])
def test_projection_then_attention(dtype, causal):
    B, N, D, H, d = 2, 200, 256, 2, 64
    pi = gen.make_projection(B, N, D, H, d, dtype, seed=4)
    x, w, b = _dev(pi.x, dtype), _dev(pi.w, dtype), _dev(pi.bias, dtype)
    q, k, v = _lib.qkv_proj(x, w, b, H, d)
    scale = 1 / math.sqrt(d)
    o, lse = _lib.fwd(q, k, v, scale, causal)
    torch.cuda.synchronize()
    # oracle: float64 projection, stored in the same format, then attention
    refs = oracle.qkv_projection(_host(pi.x, dtype), _host(pi.w, dtype), _host(pi.bias, dtype), H, d)
    stored = gen.store(dtype, *(r.astype(np.float32) for r in refs))
    q64, k64, v64 = gu.dequant(stored)
    o_ref, lse_ref = oracle.attention(q64, k64, v64, scale, causal)
    do = np.abs(gu.o_to_numpy(o) - o_ref).max()
    dl = (np.abs(lse.cpu().numpy() - lse_ref) / np.maximum(1.0, np.abs(lse_ref))).max()
    print(f"[proj] end to end max|dO| {do:.3g}, max rel dlse {dl:.3g}")
    assert do <= gu.O_TOL[dtype] and dl <= gu.LSE_TOL


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_projection_large_tile_sampled(dtype):
    """A product large enough for the 256 x 256 tile (at least four
    workgroups per CU), with a partial token tile (M = 16000) and a partial
    feature tile (3 H d = 5760); every feature of 320 sampled tokens,
    including the first and last ones, against the oracle, for both 16-bit
    types (each has its own instance of the tile)."""
    B, N, D, H, d = 4, 4000, 1024, 30, 64
    print(f"[proj] large tile B={B} N={N} D={D} H={H} d={d} {dtype}", flush=True)
    pi = gen.make_projection(B, N, D, H, d, dtype, seed=5)
    outs = _run(pi)
    rng = np.random.default_rng(6)
    toks = np.unique(np.concatenate([[0, 1, 255, 256, N - 1], rng.integers(0, N, 315)]))
    sub = gen.ProjectionInputs(dtype, np.ascontiguousarray(pi.x[:, toks]), pi.w, pi.bias, H, d)
    worst = _check(sub, [o[:, :, toks] for o in outs])
    print(f"[proj] worst error / bar {worst:.3g} over {len(toks)} tokens per batch")
