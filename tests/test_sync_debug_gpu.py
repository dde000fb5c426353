"""The barrier-checking build against the normal one, bit for bit.

``libfa_sync.so`` is built from the same sources with ``FA_SYNC_CHECK``:
full memory waits and a workgroup barrier at extra points every wave
reaches (after each tile's loads are issued, at the end of each tile, after
the Q load, before the epilogue).  There is no LDS race checker on this
platform; if a wait or barrier were missing in the normal build, the extra
ones would change what some wave reads, and with it the output.  Every
compiled forward tile shape (each dtype, with and without the causal mask),
the packed and dropout forms and the backward pass must give identical bits
from both builds.
"""
import contextlib
import math
import os

import numpy as np
import pytest
import torch

from io_aware_attention_fwd_amd import _lib, gen
from tests import gpu_util as gu
from tests.test_tiles_gpu import TILES

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    normal = _lib.load()
    sync = _lib.open_library(os.path.join(os.path.dirname(_lib.library_path()), "libfa_sync.so"))
    yield normal, sync
    _lib._LIB = normal
    os.environ.pop("FA_TILE", None)


@contextlib.contextmanager
def using(lib):
    saved = _lib._LIB
    _lib._LIB = lib
    try:
        yield
    finally:
        _lib._LIB = saved


def _same(a, b, what):
    assert a.shape == b.shape, what
    assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), f"{what} differs"


@pytest.mark.parametrize("d,tile", TILES, ids=[f"d{d}-{t}" for d, t in TILES])
@pytest.mark.parametrize("dtype", ["f16", "bf16", "fp8"])
def test_forward_tiles_identical(libs, d, tile, dtype):
    print(f"[sync] forward {tile} d={d} {dtype}", flush=True)
    x = gen.make(2, 3, 300, d, dtype, seed=21)
    q, k, v = gu.to_device(x)
    os.environ["FA_TILE"] = tile
    try:
        for causal in (False, True):
            outs = []
            for lib in libs:
                with using(lib):
                    assert _lib.fwd_tile(300, d, causal, {"f16": 0, "bf16": 1, "fp8": 2}[dtype]) == tile
                    outs.append(_lib.fwd(q, k, v, 1 / math.sqrt(d), causal))
            torch.cuda.synchronize()
            _same(outs[0][0], outs[1][0], f"O ({tile}, causal={causal})")
            _same(outs[0][1], outs[1][1], f"lse ({tile}, causal={causal})")
    finally:
        os.environ.pop("FA_TILE", None)


@pytest.mark.parametrize("B,H,N,d,dtype,causal", [(4, 8, 2000, 64, "f16", False), (4, 8, 2000, 64, "bf16", True),
                                                  (2, 4, 4100, 128, "bf16", True), (2, 8, 3000, 64, "fp8", False)])
def test_forward_defaults_larger(libs, B, H, N, d, dtype, causal):
    print(f"[sync] forward default B={B} H={H} N={N} d={d} {dtype} causal={causal}", flush=True)
    x = gen.make(B, H, N, d, dtype, seed=22)
    q, k, v = gu.to_device(x)
    outs = []
    for lib in libs:
        with using(lib):
            outs.append(_lib.fwd(q, k, v, 1 / math.sqrt(d), causal))
    torch.cuda.synchronize()
    _same(outs[0][0], outs[1][0], "O")
    _same(outs[0][1], outs[1][1], "lse")


def test_varlen_and_dropout_identical(libs):
    lengths = [0, 1, 77, 300, 1000, 129]
    for d, dtype in ((64, "f16"), (128, "bf16")):
        x, cu = gen.make_packed(lengths, 2, d, dtype, seed=23)
        q, k, v = gu.to_device(x)
        cu_t = torch.from_numpy(cu).cuda()
        for causal in (False, True):
            outs = []
            for lib in libs:
                with using(lib):
                    outs.append(_lib.fwd_varlen(q, k, v, cu_t, max(lengths), 1 / math.sqrt(d), causal))
            torch.cuda.synchronize()
            _same(outs[0][0], outs[1][0], f"varlen O d={d}")
            _same(outs[0][1], outs[1][1], f"varlen lse d={d}")
        y = gen.make(1, 2, 700, d, dtype, seed=24)
        q, k, v = gu.to_device(y)
        outs = []
        for lib in libs:
            with using(lib):
                outs.append(_lib.fwd_dropout(q, k, v, 1 / math.sqrt(d), True, 0.2, seed=99, offset=3))
        torch.cuda.synchronize()
        _same(outs[0][0], outs[1][0], f"dropout O d={d}")


# (B, H): small grids, and at d = 128 one of at least 512 workgroups of 128
# rows, where the dK/dV kernel is built for two waves per SIMD
@pytest.mark.parametrize("d,dtype,B,H", [(64, "f16", 2, 4), (64, "bf16", 2, 4), (128, "f16", 2, 4), (128, "bf16", 2, 4),
                                         (128, "bf16", 4, 32)])
@pytest.mark.parametrize("N", [300, 1000])
def test_backward_identical(libs, d, dtype, B, H, N):
    print(f"[sync] backward B={B} H={H} d={d} {dtype} N={N}", flush=True)
    x = gen.make(B, H, N, d, dtype, seed=25)
    g = gen.make(B, H, N, d, dtype, seed=26)
    q, k, v = gu.to_device(x)
    do = gu.to_device(g)[0]
    for causal in (False, True):
        o, lse = _lib.fwd(q, k, v, 1 / math.sqrt(d), causal)
        outs = []
        for lib in libs:
            with using(lib):
                outs.append(_lib.bwd(q, k, v, o, lse, do, 1 / math.sqrt(d), causal))
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), outs[0], outs[1]):
            _same(a, b, f"{name} causal={causal}")
