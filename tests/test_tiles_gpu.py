"""Every compiled tile shape of the forward kernel against the oracle.

The library picks one shape per call (head dimension, dtype, mask, N); the
``FA_TILE`` environment variable, read on every call, selects any other
shape compiled for the call's head dimension.  Each shape runs here on a
ragged N (several query and key tiles plus a partial one) for every dtype and
mask, at the forward pass's tolerances, and on lengths shorter than one
tile.  Shapes are parametrized per head dimension from the variant table, and
every case first asks the library (``fa_fwd_tile``) which shape the call will
run, so a request that silently fell back to the default would fail.
"""
import math
import os
import re

import numpy as np
import pytest
import torch

from io_aware_attention_fwd_amd import _lib, gen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_DT = {"f16": _lib.FA_DTYPE_F16, "bf16": _lib.FA_DTYPE_BF16, "fp8": _lib.FA_DTYPE_FP8_E4M3}


def _compiled_tiles():
    src = open(os.path.join(ROOT, "io_aware_attention_fwd_amd", "csrc", "fa_variants.h")).read()
    body = re.search(r"kVariants\[\] = \{(.*?)\};", src, re.S).group(1)
    tiles = ["x".join(t.replace(" ", "").split(",")) for t in re.findall(r"\{([\d,\s]+)\}", body)]
    d64 = {int(i) for i in re.findall(r"v == (\d+)", re.search(r"d64_only\(int v\) \{(.*?)\}", src).group(1))}
    d128 = {int(i) for i in re.findall(r"v == (\d+)", re.search(r"d128_only\(int v\) \{(.*?)\}", src).group(1))}
    return [(d, t) for d in (64, 128) for i, t in enumerate(tiles)
            if not (i in d64 and d != 64) and not (i in d128 and d != 128)]


TILES = _compiled_tiles()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()
    yield
    os.environ.pop("FA_TILE", None)


def _run_tile(tile, x, d, dtype, scale):
    B, H, N, _ = x.shape
    os.environ["FA_TILE"] = tile
    try:
        for causal in (False, True):
            ran = _lib.fwd_tile(N, d, causal, _DT[dtype])
            assert ran == tile, f"FA_TILE={tile} requested, the library runs {ran}"
            o, lse = gu.run_gpu(x, scale, causal)
            gu.compare(x, gu.o_to_numpy(o), lse.cpu().numpy().astype(np.float64), scale, causal)
    finally:
        os.environ.pop("FA_TILE", None)


@pytest.mark.parametrize("d,tile", TILES, ids=[f"d{d}-{t}" for d, t in TILES])
@pytest.mark.parametrize("dtype", ["f16", "bf16", "fp8"])
def test_tile_parity(d, tile, dtype):
    B, H, N = 1, 2, 300
    print(f"[tile] {tile} {dtype} d={d} N={N}", flush=True)
    x = gen.make(B, H, N, d, dtype, seed=11)
    _run_tile(tile, x, d, dtype, 1 / math.sqrt(d))


@pytest.mark.parametrize("d,tile", TILES, ids=[f"d{d}-{t}" for d, t in TILES])
@pytest.mark.parametrize("N", [1, 17, 100])
def test_tile_short_sequences(d, tile, N):
    """Lengths below one key tile and one wave's rows: most waves of the
    workgroup, and all but the first rows of the first, lie past N."""
    B, H = 2, 3
    dtype = "f16" if d == 64 else "bf16"
    print(f"[tile] {tile} {dtype} d={d} N={N}", flush=True)
    x = gen.make(B, H, N, d, dtype, seed=12)
    _run_tile(tile, x, d, dtype, 1 / math.sqrt(d))
