"""GPU parity of the backward pass ``fa_bwd`` against the float64 oracle.

The GPU pass runs the library's forward to get O and lse, then ``fa_bwd``;
the oracle differentiates the forward definition directly from Q, K, V and
dO (``oracle.attention_backward_slice``).  Bar, per tensor and slice:
max |g_gpu - g_ref| <= TOL * max(max |g_ref|, 1e-3), with TOL = 1e-2 for
binary16 and 4e-2 for bfloat16.  The floor only matters where the exact
gradient vanishes (dQ and dK of a one-key slice are zero, since dS sums to
zero along each row); the inputs are O(1), so 1e-3 is far below any real
gradient.  The error sources are the 16-bit rounding of P and dS before the
matrix products, of the stored O (through rowsum(dO * O)) and of
the outputs, each a relative 2^-11 (binary16) or 2^-8 (bfloat16) per
element; the bar is about ten such units of the tensor's largest gradient.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from io_aware_attention_fwd_amd import _lib, gen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

TOL = {"f16": 1e-2, "bf16": 4e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()


def _grads(B, H, N, d, dtype, causal, scale, seed=0):
    x = gen.make(B, H, N, d, dtype, seed=seed)
    g = gen.make(B, H, N, d, dtype, seed=seed + 100)  # dO: the first tensor of another seeded draw
    q, k, v = gu.to_device(x)
    do = gu.to_device(g)[0]
    o, lse = _lib.fwd(q, k, v, scale, causal)
    dq, dk, dv = _lib.bwd(q, k, v, o, lse, do, scale, causal)
    torch.cuda.synchronize()
    host = lambda t: t.float().cpu().numpy().astype(np.float64)
    return x, g, host(dq), host(dk), host(dv)


def _check(x, g, dq, dk, dv, scale, causal, slices):
    tol = TOL[x.dtype]
    worst = 0.0
    for b, h in slices:
        q, k, v = gu.dequant(x, b, h)
        do = oracle.dequantize(g.q[b, h], g.dtype, 1.0)
        refs = oracle.attention_backward_slice(q, k, v, do, scale, causal)
        for name, mine, ref in zip(("dQ", "dK", "dV"), (dq[b, h], dk[b, h], dv[b, h]), refs):
            assert np.isfinite(mine).all(), (name, b, h)
            mag = max(np.abs(ref).max(), 1e-3)
            err = np.abs(mine - ref).max() / mag
            assert err <= tol, f"{name} slice {(b, h)}: max|d|/max|ref| = {err:.3g} > {tol}"
            worst = max(worst, err)
    return worst


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_parity(dtype, d, causal):
    B, H, N = 1, 2, 300
    print(f"[bwd] B={B} H={H} N={N} d={d} {dtype} causal={causal}", flush=True)
    scale = 1 / math.sqrt(d)
    x, g, dq, dk, dv = _grads(B, H, N, d, dtype, causal, scale)
    worst = _check(x, g, dq, dk, dv, scale, causal, [(0, 0), (0, 1)])
    print(f"[bwd] worst normalised error {worst:.3g}")


@pytest.mark.parametrize("N", [1, 2, 17, 64, 65, 127, 129, 1000])
def test_bwd_ragged_lengths(N):
    print(f"[bwd] ragged N={N}", flush=True)
    for dtype, d, causal in (("f16", 64, True), ("bf16", 128, False)):
        scale = 1 / math.sqrt(d)
        x, g, dq, dk, dv = _grads(1, 2, N, d, dtype, causal, scale, seed=N)
        _check(x, g, dq, dk, dv, scale, causal, [(0, 0), (0, 1)])


@pytest.mark.parametrize("scale", [0.0, -0.2, 0.9])
def test_bwd_scale_values(scale):
    print(f"[bwd] scale={scale}", flush=True)
    x, g, dq, dk, dv = _grads(1, 2, 200, 64, "f16", True, scale, seed=3)
    _check(x, g, dq, dk, dv, scale, True, [(0, 0), (0, 1)])


@pytest.mark.parametrize("d,dtype,causal", [(64, "bf16", True), (128, "bf16", True), (64, "f16", False)])
def test_bwd_larger_sampled(d, dtype, causal):
    B, H, N = 2, 8, 2048
    print(f"[bwd] B={B} H={H} N={N} d={d} {dtype} causal={causal}", flush=True)
    scale = 1 / math.sqrt(d)
    x, g, dq, dk, dv = _grads(B, H, N, d, dtype, causal, scale, seed=9)
    worst = _check(x, g, dq, dk, dv, scale, causal, oracle.slice_sample(B, H, count=4))
    print(f"[bwd] worst normalised error {worst:.3g}")


# (B, H, N, dtype, causal, slices checked).  At d = 128 the dK/dV kernel is
# built for two waves per SIMD once the grid has at least 512 workgroups of
# 128 rows (two per CU of the 256); every case here reaches that build, N =
# 1000 with a ragged last block, the last at the shape its benchmark figures
# are quoted on.
LARGE_D128 = [(2, 16, 2048, "bf16", False, 4), (2, 16, 2048, "bf16", True, 4), (2, 16, 2048, "f16", False, 4),
              (2, 16, 2048, "f16", True, 4), (4, 32, 1000, "bf16", True, 4), (4, 32, 1000, "f16", False, 4),
              (4, 32, 8192, "bf16", False, 2)]


@pytest.mark.parametrize("B,H,N,dtype,causal,count", LARGE_D128,
                         ids=[f"B{c[0]}H{c[1]}N{c[2]}-{c[3]}-{'causal' if c[4] else 'full'}" for c in LARGE_D128])
def test_bwd_d128_large_grid(B, H, N, dtype, causal, count):
    d = 128
    assert -(-N // 128) * B * H >= 512  # the two-waves-per-SIMD dK/dV build runs
    print(f"[bwd] d=128 large grid B={B} H={H} N={N} {dtype} causal={causal}", flush=True)
    scale = 1 / math.sqrt(d)
    x, g, dq, dk, dv = _grads(B, H, N, d, dtype, causal, scale, seed=21)
    worst = _check(x, g, dq, dk, dv, scale, causal, oracle.slice_sample(B, H, count=count))
    print(f"[bwd] worst normalised error {worst:.3g}")
