"""Every compiled tile shape of the forward kernel against the oracle.

The library picks one shape per call (head dimension, dtype, mask, N); the
``FA_TILE`` environment variable, read on every call, selects any other
compiled shape.  Each shape runs here on a ragged N (several query and key
tiles plus a partial one) for every dtype, head dimension and mask, at the
forward pass's tolerances.
"""
import math
import os

import numpy as np
import pytest
import torch

from io_aware_attention_fwd_amd import _lib, gen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

TILES = ["32x8x64x1x2", "32x4x64x0x4", "32x4x64x0x3", "32x4x64x0x2", "64x4x64x0x2", "64x8x64x1x2", "32x16x64x1x4", "32x8x64x0x4", "64x8x32x1x2"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()
    yield
    os.environ.pop("FA_TILE", None)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("dtype", ["f16", "bf16", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
def test_tile_parity(tile, dtype, d):
    B, H, N = 1, 2, 300
    print(f"[tile] {tile} {dtype} d={d} N={N}", flush=True)
    x = gen.make(B, H, N, d, dtype, seed=11)
    scale = 1 / math.sqrt(d)
    os.environ["FA_TILE"] = tile
    try:
        for causal in (False, True):
            o, lse = gu.run_gpu(x, scale, causal)
            gu.compare(x, gu.o_to_numpy(o), lse.cpu().numpy().astype(np.float64), scale, causal)
    finally:
        os.environ.pop("FA_TILE", None)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 17, 100])
def test_tile_short_sequences(tile, d, N):
    """Lengths below one key tile and one wave's rows: most waves of the
    workgroup, and all but the first rows of the first, lie past N."""
    B, H = 2, 3
    dtype = "f16" if d == 64 else "bf16"
    print(f"[tile] {tile} {dtype} d={d} N={N}", flush=True)
    x = gen.make(B, H, N, d, dtype, seed=12)
    scale = 1 / math.sqrt(d)
    os.environ["FA_TILE"] = tile
    try:
        for causal in (False, True):
            o, lse = gu.run_gpu(x, scale, causal)
            gu.compare(x, gu.o_to_numpy(o), lse.cpu().numpy().astype(np.float64), scale, causal)
    finally:
        os.environ.pop("FA_TILE", None)
