"""GPU parity of the packed variable-length entry point ``fa_fwd_varlen``.

Sequences of different lengths are packed back to back ([total, H, d], lse
[H, total]); each (sequence, head) is compared element by element with the
float64 oracle on that sequence's rows, to the same bars as the dense path:
max |O_gpu - O_ref| <= 1e-2 (f16), 2e-2 (bf16), 6e-2 (fp8, in value units),
|lse_gpu - lse_ref| <= 1e-3 * max(1, |lse_ref|).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from io_aware_attention_fwd_amd import _lib, gen
from tests import gpu_util as gu
from tests.test_tiles_gpu import TILES  # (d, tile) of every shape compiled for d

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()


def _dev(x: gen.Inputs):
    return gu.to_device(x)


def _run(x: gen.Inputs, cu: np.ndarray, max_seqlen: int, scale: float, causal: bool, poison=True):
    q, k, v = _dev(x)
    total, H, d = q.shape
    o_dtype = torch.bfloat16 if x.dtype == "fp8" else q.dtype
    out = torch.full((total, H, d), float("nan") if poison else 0.0, dtype=o_dtype, device="cuda")
    lse = torch.full((H, total), float("nan") if poison else 0.0, dtype=torch.float32, device="cuda")
    cu_t = torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    _lib.fwd_varlen(q, k, v, cu_t, max_seqlen, scale, causal, out=out, lse=lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _compare(x, cu, o, lse, scale, causal, sequences=None, heads=None, o_scale=1.0):
    """Oracle per (sequence, head); returns (max |dO|, max rel dlse)."""
    H = x.q.shape[1]
    qd = oracle.dequantize(x.q, x.dtype, x.descale["q"])
    kd = oracle.dequantize(x.k, x.dtype, x.descale["k"])
    vd = oracle.dequantize(x.v, x.dtype, x.descale["v"])
    tol = gu.O_TOL[x.dtype]
    worst_o = worst_l = 0.0
    seqs = range(len(cu) - 1) if sequences is None else sequences
    for b in seqs:
        r0, r1 = int(cu[b]), int(cu[b + 1])
        for h in (range(H) if heads is None else heads):
            o_ref, lse_ref = oracle.attention_slice(qd[r0:r1, h], kd[r0:r1, h], vd[r0:r1, h], scale, causal)
            if r1 == r0:
                continue
            og = o[r0:r1, h] * o_scale
            assert np.isfinite(og).all() and np.isfinite(lse[h, r0:r1]).all(), (b, h)
            do = np.abs(og - o_ref).max()
            dl = (np.abs(lse[h, r0:r1] - lse_ref) / np.maximum(1.0, np.abs(lse_ref))).max()
            assert do <= tol, f"sequence {b} head {h}: max|dO| = {do:.3g} > {tol}"
            assert dl <= gu.LSE_TOL, f"sequence {b} head {h}: max rel dlse = {dl:.3g}"
            worst_o, worst_l = max(worst_o, do), max(worst_l, dl)
    return worst_o, worst_l


# Mixed lengths: single rows, an empty sequence, tile-edge lengths and tails.
LENGTHS = [1, 0, 65, 200, 17, 64, 1000, 3, 129]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_parity(dtype, d, causal):
    print(f"[varlen] {dtype} d={d} causal={causal} lengths={LENGTHS}", flush=True)
    x, cu = gen.make_packed(LENGTHS, 3, d, dtype, seed=1)
    scale = 1 / math.sqrt(d)
    o, lse = _run(x, cu, max(LENGTHS), scale, causal)
    do, dl = _compare(x, cu, o, lse, scale, causal)
    print(f"[varlen] max|dO|={do:.3g} max rel dlse={dl:.3g}")


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_fp8(causal):
    # fa_fwd_varlen takes fp8 codes with descales of 1: fold the Q and K
    # descales into the scale and rescale O by the V descale for comparison
    print(f"[varlen] fp8 causal={causal}", flush=True)
    x, cu = gen.make_packed(LENGTHS, 2, 64, "fp8", seed=2)
    scale = 1 / 8
    eff = scale * x.descale["q"] * x.descale["k"]
    o, lse = _run(x, cu, max(LENGTHS), eff, causal)
    _compare(x, cu, o, lse, scale, causal, o_scale=x.descale["v"])


@pytest.mark.parametrize("d,dtype,causal", [(64, "bf16", True), (128, "f16", False)])
def test_varlen_equal_lengths_match_dense(d, dtype, causal):
    """The same problem through fa_fwd (dense) and fa_fwd_varlen (packed)
    gives identical bits when both run the same tile shape and walk the keys
    in the same order: only the addressing differs.  (Their default shapes may
    differ: packed batches keep 128-row workgroups.)  FA_TILE pins both calls
    to the packed default.  With the causal mask the dense grid pairs query
    tiles and walks the lower tile of each pair (tiles below n/2 of a slice's
    n) from its diagonal down to key 0, so those rows differ from the packed
    path's by the order of the sums alone: they are held to the oracle bars."""
    print(f"[varlen] equal lengths vs dense d={d} {dtype} causal={causal}", flush=True)
    B, H, N = 4, 4, 300
    x, cu = gen.make_packed([N] * B, H, d, dtype, seed=3)
    os.environ["FA_TILE"] = "32x4x64x0x4" if d == 64 else "32x4x64x0x2"
    try:
        o, lse = _run(x, cu, N, 0.1, causal)
        q, k, v = _dev(x)
        dense = lambda t: t.reshape(B, N, H, d).permute(0, 2, 1, 3).contiguous()
        od, ld = _lib.fwd(dense(q), dense(k), dense(v), 0.1, causal)
        torch.cuda.synchronize()
    finally:
        os.environ.pop("FA_TILE", None)
    od = od.float().cpu().numpy().astype(np.float64)
    ld = ld.cpu().numpy().astype(np.float64)
    o = o.reshape(B, N, H, d).transpose(0, 2, 1, 3)
    lse = lse.reshape(H, B, N).transpose(1, 0, 2)
    split = (math.ceil(N / 128) // 2) * 128 if causal else 0  # rows of the tiles walked down (dense)
    assert np.array_equal(o[:, :, split:], od[:, :, split:])
    assert np.array_equal(lse[:, :, split:], ld[:, :, split:])
    if split:
        assert np.abs(o[:, :, :split] - od[:, :, :split]).max() <= gu.O_TOL[dtype]
        dl = np.abs(lse[:, :, :split] - ld[:, :, :split]) / np.maximum(1.0, np.abs(ld[:, :, :split]))
        assert dl.max() <= gu.LSE_TOL


def test_varlen_inconsistent_offsets_skip_sequences():
    """Offset pairs that decrease, run past total or exceed max_seqlen make
    their sequence empty: its rows keep their old contents, the others are
    computed, nothing is touched outside the buffers."""
    print("[varlen] inconsistent offsets", flush=True)
    H, d, total = 2, 64, 100
    x, _ = gen.make_packed([total], H, d, "f16", seed=4)
    cu = np.array([0, 40, 30, 100, 500], np.int32)  # [0,40) ok; 40->30 decreasing; 30->100 longer than 64; 100->500 past total
    o, lse = _run(x, cu, 64, 0.125, True)
    _compare(x, np.array([0, 40]), o, lse, 0.125, True)
    assert np.isnan(o[40:]).all() and np.isnan(lse[:, 40:]).all()


def test_varlen_no_rows():
    q = torch.zeros((1, 2, 64), dtype=torch.float16, device="cuda")
    out = torch.zeros_like(q)
    lse = torch.zeros((2, 1), device="cuda")
    cu_t = torch.zeros(3, dtype=torch.int32, device="cuda")
    rc = _lib.fa_fwd_varlen(q.data_ptr(), q.data_ptr(), q.data_ptr(), out.data_ptr(), lse.data_ptr(), cu_t.data_ptr(),
                            2, 2, 0, 1, 64, 0.1, 0, _lib.FA_DTYPE_F16, None)
    assert rc == 0


@pytest.mark.parametrize("d,dtype,causal", [(128, "bf16", True), (64, "f16", False)])
def test_varlen_long_sequences_sampled(d, dtype, causal):
    """Long and short sequences in one batch; the oracle checks a sample of
    (sequence, head) pairs, every row of each."""
    lengths = [8192, 1, 4096, 3000, 777, 8191]
    H = 16
    print(f"[varlen] long d={d} {dtype} causal={causal} lengths={lengths}", flush=True)
    x, cu = gen.make_packed(lengths, H, d, dtype, seed=5)
    scale = 1 / math.sqrt(d)
    o, lse = _run(x, cu, max(lengths), scale, causal)
    do, dl = _compare(x, cu, o, lse, scale, causal, sequences=[0, 1, 5], heads=[0, 15])
    print(f"[varlen] max|dO|={do:.3g} max rel dlse={dl:.3g}")


# Every compiled tile shape (FA_TILE) on the mixed-length batch: the packed
# addressing (sequence bounds, empty query tiles, rows past a sequence's end)
# is shared by all of them.
@pytest.mark.parametrize("d,tile", TILES, ids=[f"d{d}-{t}" for d, t in TILES])
def test_varlen_every_tile(d, tile):
    dtype = "f16" if d == 64 else "bf16"
    print(f"[varlen] tile {tile} d={d} {dtype}", flush=True)
    x, cu = gen.make_packed(LENGTHS, 2, d, dtype, seed=13)
    scale = 1 / math.sqrt(d)
    os.environ["FA_TILE"] = tile
    try:
        for causal in (False, True):
            ran = _lib.fwd_tile(max(LENGTHS), d, causal, {"f16": 0, "bf16": 1}[dtype], _lib.FA_TILE_VARLEN)
            assert ran == tile, f"FA_TILE={tile} requested, the library runs {ran}"
            o, lse = _run(x, cu, max(LENGTHS), scale, causal)
            _compare(x, cu, o, lse, scale, causal)
    finally:
        os.environ.pop("FA_TILE", None)
