"""Seeded synthetic inputs for the attention forward pass.

This module only *draws and stores* inputs; it does none of the attention
arithmetic.  Both the GPU path (through the tests and the benchmark) and the
CPU oracle are fed from it, so the two sides always see the same bytes.

Workload shape follows the forward-time tables of the benchmark page
("Optimization Flash Attention 基准测试", tables for A100 80GB and H100 80GB:
batch=8, heads=32, dim=64, sequence lengths 512..8192).  Values are i.i.d.
N(0, 1) drawn from ``numpy.random.default_rng(seed)`` in float32, in the order
Q, then K, then V, each of shape [B, H, N, d], and then rounded to the storage
format:

* ``f16``  -- IEEE binary16, round-to-nearest-even (numpy ``astype``).
* ``bf16`` -- bfloat16, round-to-nearest-even, returned as its uint16 bit
  pattern because numpy has no bfloat16 type.
* ``fp8``  -- OCP FP8 E4M3 ("e4m3fn": max 448, no infinities, 0x7F/0xFF NaN)
  with one float32 scale per tensor, ``s = amax|X| / 448``.  The code is
  ``RNE(clamp(X / s, -448, 448))``.  The clamp is explicit because a plain
  float32 -> e4m3fn cast does not saturate (1000 becomes NaN).  ``s`` is the
  descale the kernel and the oracle multiply codes by.

Storage arrays are numpy, C-contiguous, [B, H, N, d] with d innermost.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f16", "bf16", "fp8")
E4M3_MAX = 448.0


@dataclass
class Inputs:
    """Stored inputs of one attention call.

    ``q``, ``k``, ``v`` hold the storage bits: ``np.float16`` for f16,
    ``np.uint16`` (bfloat16 bit patterns) for bf16, ``np.uint8`` (e4m3 codes)
    for fp8.  ``descale`` maps 'q'/'k'/'v' to the float32 per-tensor scale
    (1.0 for f16/bf16).
    """

    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    descale: dict = field(default_factory=lambda: {"q": 1.0, "k": 1.0, "v": 1.0})

    @property
    def shape(self):
        return self.q.shape


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs here are finite draws, so no NaN handling is needed; a NaN input
    raises rather than being silently rounded.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.isfinite(x).all():
        raise ValueError("bf16 rounding expects finite inputs")
    # finite float32 bit patterns stay below 2^32 after adding 0x8000, so
    # uint32 arithmetic cannot wrap; work in chunks to bound temporaries
    flat = x.reshape(-1)
    out = np.empty(flat.shape, np.uint16)
    step = 1 << 24
    for i in range(0, flat.size, step):
        bits = flat[i:i + step].view(np.uint32).copy()
        lsb = (bits >> 16) & 1
        bits += 0x7FFF
        bits += lsb
        bits >>= 16
        out[i:i + step] = bits
    return out.reshape(x.shape)


def quantize_e4m3(x: np.ndarray) -> tuple[np.ndarray, float]:
    """Per-tensor OCP e4m3 quantisation: returns (uint8 codes, float32 scale)."""
    import torch  # the RNE float32 -> e4m3fn conversion is torch's

    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = float(np.abs(x).max()) if x.size else 0.0
    s = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
    y = np.clip(x / s, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes.copy(), float(s)


def draw_normal(B: int, H: int, N: int, d: int, seed: int = 0):
    """Three float32 [B,H,N,d] arrays (Q, K, V) of i.i.d. N(0,1) draws."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    q = rng.standard_normal(size=shape, dtype=np.float32)
    k = rng.standard_normal(size=shape, dtype=np.float32)
    v = rng.standard_normal(size=shape, dtype=np.float32)
    return q, k, v


def store(dtype: str, q32: np.ndarray, k32: np.ndarray, v32: np.ndarray) -> Inputs:
    """Round float32 Q, K, V to the storage format ``dtype``."""
    if dtype == "f16":
        return Inputs("f16", q32.astype(np.float16), k32.astype(np.float16), v32.astype(np.float16))
    if dtype == "bf16":
        return Inputs("bf16", f32_to_bf16_bits(q32), f32_to_bf16_bits(k32), f32_to_bf16_bits(v32))
    if dtype == "fp8":
        qc, sq = quantize_e4m3(q32)
        kc, sk = quantize_e4m3(k32)
        vc, sv = quantize_e4m3(v32)
        return Inputs("fp8", qc, kc, vc, {"q": sq, "k": sk, "v": sv})
    raise ValueError(f"unknown dtype {dtype!r}; expected one of {DTYPES}")


def make(B: int, H: int, N: int, d: int, dtype: str, seed: int = 0) -> Inputs:
    """The standard workload: N(0,1) draws from ``seed`` stored as ``dtype``."""
    q, k, v = draw_normal(B, H, N, d, seed)
    return store(dtype, q, k, v)


def make_packed(lengths, H: int, d: int, dtype: str, seed: int = 0):
    """Sequences of the given lengths packed back to back: Q, K, V of shape
    [total, H, d] (N(0,1) draws from ``seed`` in the order Q, K, V, stored as
    ``dtype``) and the B+1 row offsets as an int32 array."""
    lengths = [int(n) for n in lengths]
    if any(n < 0 for n in lengths):
        raise ValueError("sequence lengths must be >= 0")
    total = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal(size=(total, H, d), dtype=np.float32) for _ in range(3))
    return store(dtype, q, k, v), cu


def length_mix(count: int, lo: int, hi: int, seed: int = 0):
    """``count`` sequence lengths drawn uniformly from [lo, hi] (inclusive)."""
    return [int(n) for n in np.random.default_rng(seed).integers(lo, hi + 1, size=count)]


def structured(B: int, H: int, N: int, d: int, dtype: str, period: int = 64) -> Inputs:
    """Inputs whose exact output is known row by row.

    Q = 0 (every score is 0, so each query averages the values of the keys it
    may see), K = N(0,1) draws (seed 1), and V[j, c] = ((j // period) + c) mod 7,
    small integers that every storage format holds exactly (fp8 with descale 1).
    A dropped or duplicated block of ``period`` keys changes the average of
    every row that sees it.
    """
    rng = np.random.default_rng(1)
    k32 = rng.standard_normal(size=(B, H, N, d), dtype=np.float32)
    q32 = np.zeros((B, H, N, d), np.float32)
    j = np.arange(N)[:, None]
    c = np.arange(d)[None, :]
    v32 = np.broadcast_to((((j // period) + c) % 7).astype(np.float32), (B, H, N, d)).copy()
    if dtype == "fp8":
        import torch

        enc = lambda a: torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
        return Inputs("fp8", enc(q32), enc(k32), enc(v32), {"q": 1.0, "k": 1.0, "v": 1.0})
    return store(dtype, q32, k32, v32)


def onehot_blocks(B: int, H: int, N: int, d: int, dtype: str, block: int = 8) -> Inputs:
    """Full-size inputs whose exact output is known for every row of every slice.

    Q = 0 (every score is 0 whatever K holds, so each query averages the
    values of the keys it may see), K = small integers in [-3, 3] (seed 2),
    and V one-hot by key block: V[b, h, j, c] = 1 if (j // block + b*H + h)
    mod d == c, else 0.  Every value is exact in every storage format (fp8
    with descale 1).  A dropped, duplicated or misplaced block of ``block``
    keys moves the visible-key count of one column, and a slice read in
    place of another shifts the columns.
    """
    rng = np.random.default_rng(2)
    k32 = rng.integers(-3, 4, size=(B, H, N, d), dtype=np.int8).astype(np.float32)
    q32 = np.zeros((B, H, N, d), np.float32)
    col = (np.arange(N)[None, None, :] // block + np.arange(B * H).reshape(B, H, 1)) % d  # [B, H, N]
    v32 = (col[..., None] == np.arange(d)).astype(np.float32)
    if dtype == "fp8":
        # E4M3 codes: 0 -> 0x00, 1 -> 0x38; the small integers of K through the encoder
        import torch

        enc = lambda a: torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
        return Inputs("fp8", np.zeros(q32.shape, np.uint8), enc(k32), np.where(v32 > 0, 0x38, 0).astype(np.uint8),
                      {"q": 1.0, "k": 1.0, "v": 1.0})
    return store(dtype, q32, k32, v32)


@dataclass
class ProjectionInputs:
    """Stored inputs of one QKV projection: x [B, N, D], w [3 H d, D] and
    bias [3 H d] in the storage format of ``dtype`` (f16 or bf16 bits as in
    ``Inputs``)."""

    dtype: str
    x: np.ndarray
    w: np.ndarray
    bias: np.ndarray
    H: int
    d: int


def make_projection(B: int, N: int, D: int, H: int, d: int, dtype: str, seed: int = 0) -> ProjectionInputs:
    """x ~ N(0, 1), weight ~ N(0, 1/D) (a linear layer's usual initial scale,
    so that projected values are of order 1) and bias ~ N(0, 0.01), drawn in
    that order from ``default_rng(seed)`` in float32 and stored as ``dtype``."""
    if dtype not in ("f16", "bf16"):
        raise ValueError("the projection takes f16 or bf16")
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=(B, N, D), dtype=np.float32)
    w = rng.standard_normal(size=(3 * H * d, D), dtype=np.float32) * np.float32(1.0 / np.sqrt(D))
    bias = rng.standard_normal(size=(3 * H * d,), dtype=np.float32) * np.float32(0.1)
    if dtype == "f16":
        cast = lambda a: a.astype(np.float16)
    else:
        cast = f32_to_bf16_bits
    return ProjectionInputs(dtype, cast(x), cast(w), cast(bias), H, d)


def nbytes_kv(B: int, H: int, N: int, d: int, elem_bytes: int = 2) -> int:
    """Bytes of one K plus one V tensor of shape [B, H, N, d]."""
    return 2 * B * H * N * d * elem_bytes
