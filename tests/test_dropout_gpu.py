"""GPU parity of ``fa_fwd_dropout`` against the float64 dropout oracle.

Two kinds of check:

* Exact keep mask.  With Q = 0 every visible score is 0, so P_ij = 1/n_i
  exactly (n_i visible keys) and the kernel's probabilities are exactly 1.
  V is zero except on a window of W = m * d keys starting at key a, where
  V_j = 2^((j - a) div d) e_((j - a) mod d).  Then
      O_ic = (256 / t) / n_i * sum_k M_(i, a + c + k d) 2^k,   k < m,
  an integer (the mask bits of the window's keys in column c) times a known
  constant: rounding O_ic * n_i * t / 256 recovers the integer, and its bits
  are compared with the oracle's mask bit for bit.  The integer has m bits;
  m = 8 for binary16 outputs (11 significant bits: rounding moves an 8-bit
  integer by at most 2^-3) and 6 for bfloat16 (8 significant bits: at most
  2^-3 too).  One call per window covers all N keys.
* Random inputs against ``oracle.attention_dropout``: O within the forward
  bar scaled by 256/t (the rescale multiplies the rounding of the kept
  probabilities), lse within the forward bar (dropout does not touch it).
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()


def _mask_from_gpu(B, H, N, d, dtype, causal, p, seed, offset):
    """Recover the kernel's keep mask [B, H, N, N] (invisible keys False)."""
    m = 8 if dtype == "f16" else 6
    W = m * d
    t = oracle.keep_threshold(p)
    q = torch.zeros((B, H, N, d), dtype=_TORCH[dtype], device="cuda")
    k = torch.randn((B, H, N, d), device="cuda").to(_TORCH[dtype])
    n_i = (np.arange(N) + 1 if causal else np.full(N, N)).astype(np.float64)
    mask = np.zeros((B, H, N, N), dtype=bool)
    for a in range(0, N, W):
        keys = np.arange(a, min(N, a + W))
        vals = np.zeros((N, d), dtype=np.float64)
        vals[keys, (keys - a) % d] = 2.0 ** ((keys - a) // d)
        v = torch.from_numpy(vals).to(_TORCH[dtype]).cuda().expand(B, H, N, d).contiguous()
        o, _ = _lib.fwd_dropout(q, k, v, 1.0, causal, p, seed, offset)
        torch.cuda.synchronize()
        o = o.float().cpu().numpy().astype(np.float64)
        ints = np.rint(o * n_i[None, None, :, None] * t / 256.0).astype(np.int64)  # [B, H, N, d]
        err = np.abs(o * n_i[None, None, :, None] * t / 256.0 - ints).max()
        assert err < 0.25 and np.all((ints >= 0) & (ints < (1 << m))), f"not an integer multiple of the kept weight ({err:.3g})"
        for kk in keys:
            mask[:, :, :, kk] = (ints[:, :, :, (kk - a) % d] >> ((kk - a) // d)) & 1
    return mask


@pytest.mark.parametrize("dtype,d,N,causal,p", [
    ("f16", 64, 100, False, 0.1),
    ("f16", 64, 300, True, 0.5),
    ("f16", 64, 2048, False, 0.25),   # 64-row waves
    ("f16", 128, 1000, True, 0.1),    # ping-pong schedule
    ("bf16", 128, 260, False, 0.6),
    ("bf16", 64, 2048, False, 0.1),
    ("bf16", 64, 129, True, 1 - 1 / 256),  # t = 1: only byte 0 is kept
])
def test_dropout_mask_is_exact(dtype, d, N, causal, p):
    B, H = 2, 3
    seed, offset = 0x0123_4567_89AB_CDEF, 7
    print(f"[dropout] mask B={B} H={H} N={N} d={d} {dtype} causal={causal} p={p}", flush=True)
    got = _mask_from_gpu(B, H, N, d, dtype, causal, p, seed, offset)
    t = oracle.keep_threshold(p)
    visible = np.tril(np.ones((N, N), dtype=bool)) if causal else np.ones((N, N), dtype=bool)
    for b in range(B):
        for h in range(H):
            want = (oracle.dropout_bytes(N, N, b * H + h, seed, offset) < t) & visible
            bad = np.argwhere(got[b, h] != want)
            assert bad.size == 0, f"slice {(b, h)}: {len(bad)} mask bits differ, first at (row, key) {tuple(bad[0])}"
    frac = got.sum() / (B * H * visible.sum())
    print(f"[dropout] kept fraction {frac:.4f} (t/256 = {t / 256:.4f})")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_dropout_parity(dtype, d, causal):
    B, H, N, p = 1, 2, 300, 0.2
    seed, offset = 2024, 3
    print(f"[dropout] parity B={B} H={H} N={N} d={d} {dtype} causal={causal} p={p}", flush=True)
    x = gen.make(B, H, N, d, dtype, seed=5)
    q, k, v = gu.to_device(x)
    scale = 1 / math.sqrt(d)
    o, lse = _lib.fwd_dropout(q, k, v, scale, causal, p, seed, offset)
    torch.cuda.synchronize()
    o, lse = gu.o_to_numpy(o), lse.cpu().numpy().astype(np.float64)
    t = oracle.keep_threshold(p)
    qd, kd, vd = gu.dequant(x)
    o_ref, lse_ref = oracle.attention_dropout(qd, kd, vd, scale, causal, p, seed, offset)
    tol = gu.O_TOL[dtype] * 256 / t
    do = np.abs(o - o_ref).max()
    dl = (np.abs(lse - lse_ref) / np.maximum(1.0, np.abs(lse_ref))).max()
    print(f"[dropout] max|dO| {do:.3g} (bar {tol:.3g}), max rel dlse {dl:.3g}")
    assert do <= tol and dl <= gu.LSE_TOL


def test_dropout_larger_sampled():
    B, H, N, d, dtype, p = 2, 8, 4096, 128, "bf16", 0.1
    seed, offset = 99, 0
    print(f"[dropout] sampled B={B} H={H} N={N} d={d} {dtype} causal p={p}", flush=True)
    x = gen.make(B, H, N, d, dtype, seed=6)
    q, k, v = gu.to_device(x)
    scale = 1 / math.sqrt(d)
    o, lse = _lib.fwd_dropout(q, k, v, scale, True, p, seed, offset)
    torch.cuda.synchronize()
    o, lse = gu.o_to_numpy(o), lse.cpu().numpy().astype(np.float64)
    t = oracle.keep_threshold(p)
    slices = oracle.slice_sample(B, H, count=4)
    qd, kd, vd = gu.dequant(x)
    o_ref, lse_ref = oracle.attention_dropout(qd, kd, vd, scale, True, p, seed, offset, slices=slices)
    for b, h in slices:
        do = np.abs(o[b, h] - o_ref[b, h]).max()
        dl = (np.abs(lse[b, h] - lse_ref[b, h]) / np.maximum(1.0, np.abs(lse_ref[b, h]))).max()
        assert do <= gu.O_TOL[dtype] * 256 / t and dl <= gu.LSE_TOL, ((b, h), do, dl)


def test_dropout_rate_zero_is_fwd_bitwise():
    x = gen.make(2, 4, 777, 64, "f16", seed=7)
    q, k, v = gu.to_device(x)
    for causal in (False, True):
        o0, l0 = _lib.fwd(q, k, v, 0.125, causal)
        o1, l1 = _lib.fwd_dropout(q, k, v, 0.125, causal, 0.0, 5, 0)
        torch.cuda.synchronize()
        assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_dropout_is_a_function_of_seed_and_offset():
    x = gen.make(1, 4, 513, 128, "bf16", seed=8)
    q, k, v = gu.to_device(x)
    a, la = _lib.fwd_dropout(q, k, v, 0.09, False, 0.3, 11, 1)
    b, lb = _lib.fwd_dropout(q, k, v, 0.09, False, 0.3, 11, 1)
    c, lc = _lib.fwd_dropout(q, k, v, 0.09, False, 0.3, 11, 2)
    ref, lref = _lib.fwd(q, k, v, 0.09, False)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
    assert not torch.equal(a, c)
    # lse does not see the mask
    assert torch.allclose(la, lref, rtol=1e-6, atol=0) and torch.allclose(lc, lref, rtol=1e-6, atol=0)
