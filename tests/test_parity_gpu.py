"""GPU parity: libfa.so through the C ABI against the float64 oracle.

Tolerances (max |O_gpu - O_ref|): 1e-2 f16, 2e-2 bf16, 6e-2 fp8 (against the
oracle fed the dequantised inputs); lse within 1e-3 * max(1, |lse_ref|).
Large shapes are checked on the 8 (b, h) slices of ``oracle.slice_sample``,
every row of each.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from io_aware_attention_fwd_amd import _lib, gen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# (name, B, H, N, d, dtype, causal, scale)
CONFIGS = [
    ("c1", 1, 2, 128, 64, "f16", False, 1 / 8),
    ("c2", 8, 32, 1024, 64, "f16", False, 1 / 8),
    ("c3", 8, 32, 4096, 64, "bf16", True, 1 / 8),
    ("c4", 8, 32, 8192, 64, "fp8", False, 1 / 8),
    ("c5", 2, 16, 16384, 128, "bf16", True, 1 / math.sqrt(128)),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()


def _sampled(B, H, N):
    return None if B * H * N <= 8 * 32 * 1024 else oracle.slice_sample(B, H)


@pytest.mark.parametrize("cfg", CONFIGS, ids=[c[0] for c in CONFIGS])
def test_config_parity(cfg):
    name, B, H, N, d, dtype, causal, scale = cfg
    print(f"[parity] {name} B={B} H={H} N={N} d={d} {dtype} causal={causal}", flush=True)
    x = gen.make(B, H, N, d, dtype, seed=0)
    o, lse = gu.run_gpu(x, scale, causal)
    o_np, lse_np = gu.o_to_numpy(o), lse.cpu().numpy().astype(np.float64)
    do, dl, mag = gu.compare(x, o_np, lse_np, scale, causal, slices=_sampled(B, H, N))
    print(f"[parity] {name}: max|dO|={do:.3g} (|O_ref|max {mag:.3g}, normalised {do / mag:.3g}), max rel dlse={dl:.3g}")


ODD_N = [1, 2, 3, 15, 16, 17, 63, 64, 65, 100, 127, 128, 129, 255, 1000]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_lengths(dtype, d, causal):
    print(f"[ragged] {dtype} d={d} causal={causal}", flush=True)
    for N in ODD_N:
        x = gen.make(1, 2, N, d, dtype, seed=N)
        scale = 1 / math.sqrt(d)
        o, lse = gu.run_gpu(x, scale, causal)
        gu.compare(x, gu.o_to_numpy(o), lse.cpu().numpy().astype(np.float64), scale, causal)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_structured_closed_form(dtype, d, causal):
    """Q = 0, V[j, c] = ((j // 64) + c) mod 7: O_i is the exact mean of the visible V rows."""
    N = 1000
    x = gen.structured(1, 2, N, d, dtype, period=64)
    print(f"[structured] {dtype} d={d} causal={causal}", flush=True)
    o, lse = gu.run_gpu(x, 0.7, causal)
    o_np, lse_np = gu.o_to_numpy(o), lse.cpu().numpy().astype(np.float64)
    v = ((np.arange(N)[:, None] // 64 + np.arange(d)[None, :]) % 7).astype(np.float64)
    if causal:
        want = np.cumsum(v, axis=0) / np.arange(1, N + 1)[:, None]
        want_lse = np.log(np.arange(1, N + 1))
    else:
        want = np.tile(v.mean(axis=0), (N, 1))
        want_lse = np.full(N, np.log(N))
    for h in range(2):
        # the only error left is the rounding of O to the output format
        assert np.abs(o_np[0, h] - want).max() <= 6.0 * 2.0 ** -8
        assert np.abs(lse_np[0, h] - want_lse).max() <= 1e-5 * np.log(N)


# Binary16 at d = 64 multiplies Q by scale*log2(e) in the kernel when that
# factor lies in [2^-4, 1] (0, -0.125 and 0.5 here; a zero scale zeroes Q and
# uses the factor 1) and otherwise keeps the factor in the softmax (1.0 and
# 0.02): both paths against the oracle.
@pytest.mark.parametrize("dtype", ["f16", "bf16", "fp8"])
@pytest.mark.parametrize("scale", [0.0, -0.125, 0.5, 1.0, 0.02])
def test_scale_values(dtype, scale):
    print(f"[scale] {dtype} scale={scale}", flush=True)
    for causal in (False, True):
        x = gen.make(2, 2, 200, 64, dtype, seed=3)
        o, lse = gu.run_gpu(x, scale, causal)
        gu.compare(x, gu.o_to_numpy(o), lse.cpu().numpy().astype(np.float64), scale, causal)


def test_every_output_written_and_guards_intact():
    B, H, N, d = 2, 3, 333, 64
    x = gen.make(B, H, N, d, "f16", seed=9)
    q, k, v = gu.to_device(x)
    guard = 4096
    o_buf = torch.full((B * H * N * d + 2 * guard,), float("nan"), dtype=torch.float16, device="cuda")
    l_buf = torch.full((B * H * N + 2 * guard,), -12345.0, dtype=torch.float32, device="cuda")
    o = o_buf[guard:guard + B * H * N * d].view(B, H, N, d)
    lse = l_buf[guard:guard + B * H * N].view(B, H, N)
    _lib.fwd(q, k, v, 0.125, False, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and (lse != -12345.0).all()
    assert torch.isnan(o_buf[:guard]).all() and torch.isnan(o_buf[-guard:]).all()
    assert (l_buf[:guard] == -12345.0).all() and (l_buf[-guard:] == -12345.0).all()


def test_deterministic_bitwise():
    x = gen.make(2, 4, 777, 128, "bf16", seed=4)
    o1, l1 = gu.run_gpu(x, 0.09, True)
    o2, l2 = gu.run_gpu(x, 0.09, True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_no_device_allocation_and_nonzero_stream():
    """The library allocates nothing (no score matrix in device memory) and honours the stream."""
    x = gen.make(4, 8, 2048, 64, "f16", seed=5)
    q, k, v = gu.to_device(x)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    # the first launch loads the code object (runtime memory, not the library's)
    _lib.fwd(q, k, v, 0.125, False, out=o, lse=lse, stream=side)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    o.fill_(float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        for _ in range(3):
            _lib.fwd(q, k, v, 0.125, False, out=o, lse=lse, stream=side)
    side.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0
    gu.compare(x, gu.o_to_numpy(o), lse.cpu().numpy().astype(np.float64), 0.125, False,
               slices=[(0, 0), (3, 7), (2, 5)])


def test_lse_self_consistency_large():
    """O_i = sum_j exp(S_ij - lse_i) V_j with the GPU's own lse, on sampled rows of c2's shape."""
    x = gen.make(8, 32, 1024, 64, "f16", seed=0)
    o, lse = gu.run_gpu(x, 0.125, False)
    o_np, lse_np = gu.o_to_numpy(o), lse.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(0)
    for b, h in oracle.slice_sample(8, 32):
        q, k, v = gu.dequant(x, b, h)
        rows = rng.choice(1024, 16, replace=False)
        s = 0.125 * q[rows] @ k.T
        w = np.exp(s - lse_np[b, h, rows][:, None])
        assert np.abs(w.sum(axis=1) - 1.0).max() < 1e-3
        assert np.abs(w @ v - o_np[b, h, rows]).max() < 1e-2


@pytest.mark.parametrize("N,d,dtype,causal", [(131072, 128, "bf16", True), (65536, 64, "f16", False),
                                              (32768, 128, "f16", False), (32768, 128, "fp8", False)])
def test_long_sequences_sampled_rows(N, d, dtype, causal):
    """Long sequences (a 32 MiB slice at N = 131072, d = 128): 24 sampled rows
    per slice, the first and last included, each against the oracle on the
    keys it sees (causal row i: keys 0..i as a plain attention problem)."""
    B, H = 1, 2
    print(f"[long] N={N} d={d} {dtype} causal={causal}", flush=True)
    x = gen.make(B, H, N, d, dtype, seed=12)
    scale = 1 / math.sqrt(d)
    o, lse = gu.run_gpu(x, scale, causal)
    o_np, lse_np = gu.o_to_numpy(o), lse.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(13)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, N - 2, N - 1], rng.integers(0, N, 18)]))
    for h in range(H):
        q, k, v = gu.dequant(x, 0, h)
        for i in rows:
            n_vis = i + 1 if causal else N
            o_ref, lse_ref = oracle.attention_slice(q[i:i + 1], k[:n_vis], v[:n_vis], scale, False)
            assert np.abs(o_np[0, h, i] - o_ref[0]).max() <= gu.O_TOL[dtype], (h, i)
            assert abs(lse_np[0, h, i] - lse_ref[0]) <= gu.LSE_TOL * max(1.0, abs(lse_ref[0])), (h, i)


def _growing_scores(B, H, N, d, dtype, jumps, seed=5):
    """Q and K aligned with one shared direction so that every query's scores
    step up (in the exp2 domain, scale*log2(e)*q.k) by jumps[t] at key tile
    t (64 keys); V i.i.d. N(0,1).  The first tile sets the row references and
    the later ones exceed them by the accumulated jumps."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(d).astype(np.float32)
    u /= np.linalg.norm(u)
    scale = 1 / math.sqrt(d)
    level = np.cumsum([0.0] + list(jumps))  # exp2-domain offset of each tile
    t = level[np.minimum(np.arange(N) // 64, len(level) - 1)] / (scale * math.log2(math.e) * 4.0)
    q = (4.0 * u + 0.3 * rng.standard_normal((B, H, N, d))).astype(np.float32)
    k = (t[:, None] * u + 0.3 * rng.standard_normal((B, H, N, d))).astype(np.float32)
    v = rng.standard_normal((B, H, N, d)).astype(np.float32)
    return gen.store(dtype, q, k, v), scale


# jumps per key tile, in the exp2 domain (tile maxima sit ~3 above them with
# the noise): 7 keeps every later tile's partial sums below 2^15, so the tiles
# are accepted against the first tile's references with probabilities up to
# ~2^10 (the old rule rescaled above 2^8); 30 leaves the 16-bit range (the
# tile's maxima are taken and the rows rescaled); the ramp and the mix do both
# along the sequence.
@pytest.mark.parametrize("jumps", [[7.0], [30.0], [12.0] * 9, [3.0, 7.0, 25.0, 0.0, 40.0]],
                         ids=["step7", "step30", "ramp12", "mixed"])
@pytest.mark.parametrize("dtype,d", [("f16", 64), ("bf16", 64), ("fp8", 64), ("f16", 128), ("bf16", 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_growing_scores_rescale(jumps, dtype, d, causal):
    B, H, N = 1, 2, 640
    print(f"[growing] jumps={jumps} {dtype} d={d} causal={causal}", flush=True)
    x, scale = _growing_scores(B, H, N, d, dtype, jumps)
    o, lse = gu.run_gpu(x, scale, causal)
    gu.compare(x, gu.o_to_numpy(o), lse.cpu().numpy().astype(np.float64), scale, causal)


# The mirror image for the causal grid, whose workgroups walk their shorter
# query tile's keys down from the diagonal: scores fall along the keys, so the
# first tiles such a walk visits hold the smallest scores and every tile
# further down raises the rows' maxima (by 7: accepted against the earlier
# references; by 30: rescaled; the mix: both, and tiles that lower them).
# N = 1189 gives an odd number of query tiles and a ragged last one for
# 128-, 256- and 512-row workgroups alike (one workgroup runs a lone middle
# tile).
@pytest.mark.parametrize("jumps", [[-7.0] * 19, [-30.0], [-3.0, -7.0, -25.0, 0.0, -40.0, 9.0]],
                         ids=["fall7", "fall30", "mixed"])
@pytest.mark.parametrize("dtype,d", [("f16", 64), ("bf16", 64), ("fp8", 64), ("f16", 128), ("bf16", 128)])
def test_falling_scores_downward_walk(jumps, dtype, d):
    B, H, N = 1, 2, 1189
    print(f"[falling] jumps={jumps} {dtype} d={d} tile={_lib.fwd_tile(N, d, True, {'f16': 0, 'bf16': 1, 'fp8': 2}[dtype])}",
          flush=True)
    x, scale = _growing_scores(B, H, N, d, dtype, jumps)
    o, lse = gu.run_gpu(x, scale, True)
    gu.compare(x, gu.o_to_numpy(o), lse.cpu().numpy().astype(np.float64), scale, True)


@pytest.mark.parametrize("cfg", CONFIGS[1:], ids=[c[0] for c in CONFIGS[1:]])
def test_full_size_exact_onehot(cfg):
    """The configurations at full size, in the launch configuration the
    benchmark times (default tile, whole grid), on inputs with an exact answer
    for every row (``gen.onehot_blocks``: Q = 0, V one-hot by 8-key block,
    shifted per slice).  lse must be ln(visible keys) on every row of every
    slice: one key tile dropped or counted twice moves it by ln(N/(N-64)),
    1/128 at N = 8192, which random inputs hide inside the 1e-3 bar.  O must be
    the visible-key count of each column over the visible keys, to the output
    rounding, on the 8 sampled slices: a lost or repeated 8-key block, or a
    slice read in place of another, moves a column."""
    name, B, H, N, d, dtype, causal, scale = cfg
    tile = _lib.fwd_tile(N, d, causal, {"f16": 0, "bf16": 1, "fp8": 2}[dtype])
    print(f"[onehot] {name} B={B} H={H} N={N} d={d} {dtype} causal={causal} tile={tile}", flush=True)
    x = gen.onehot_blocks(B, H, N, d, dtype, block=8)
    o, lse = gu.run_gpu(x, scale, causal)
    n_vis = np.arange(1, N + 1, dtype=np.float64) if causal else np.full(N, float(N))
    lse_np = lse.cpu().numpy().astype(np.float64)
    err_l = np.abs(lse_np - np.log(n_vis)[None, None, :]).max()
    assert err_l <= 1e-5 * math.log(N), f"max |lse - ln(visible keys)| = {err_l:.3g}"
    worst = 0.0
    for b, h in oracle.slice_sample(B, H):
        v = oracle.dequantize(x.v[b, h], x.dtype, 1.0)
        counts = np.cumsum(v, axis=0) if causal else np.broadcast_to(v.sum(axis=0), (N, d))
        want = counts / n_vis[:, None]
        got = o[b, h].float().cpu().numpy().astype(np.float64)
        err = np.abs(got - want)
        # one rounding to bfloat16 / binary16 (relative 2^-9 / 2^-12) of a value in [0, 1]
        assert (err <= 2.0 ** -8 * want + 1e-6).all(), f"slice {(b, h)}: max|dO| = {err.max():.3g}"
        worst = max(worst, float(err.max()))
    print(f"[onehot] {name}: max|lse - ln n| = {err_l:.3g}, max|dO| on sampled slices = {worst:.3g}")
