"""Attention forward with dropout on the probabilities, in float64.

Test infrastructure only (see the package docstring).

Passage: the tuning dict of page "从RTX 3090到H100：FlashAttention在NVIDIA各代GPU
架构上的性能全景分析", section 3.2, sets a dropout rate of 0.1 and remarks that a
non-zero rate needs special handling.  The pages say neither where dropout
acts nor which random numbers drive it.  The readings taken here:

1. Where: on the normalised probabilities, after the softmax and before the
   weighted sum.  With keep mask M (entries 0 or 1) and keep probability
   kappa,   O_i = sum_j (P_ij * M_ij / kappa) V_j.
   The softmax normaliser and the logsumexp are those of the full row: the
   returned lse is exactly the one without dropout.
2. Keep decision: every score draws one byte u_ij in 0..255 and is kept iff
   u_ij < t, where t = floor(256 * (1 - p) + 1/2) for the drop rate p (a
   binary32 value; the expression is exact in binary64).  t must be at least
   1.  The keep probability is then kappa = t / 256 exactly, and kept
   probabilities are scaled by 256 / t, so that the expected output equals
   the output without dropout.
3. Generator: Philox4x32-10, the counter-based generator of Salmon, Moraes,
   Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC 2011).
   A 128-bit counter (c0, c1, c2, c3) and a 64-bit key (k0, k1) go through
   ten rounds; one round, with M0 = 0xD2511F53 and M1 = 0xCD9E8D57, maps the
   counter to
       (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))
   (hi/lo: upper/lower 32 bits of the 64-bit product), and between rounds
   the key grows by (0x9E3779B9, 0xBB67AE85) modulo 2^32.
4. Which byte belongs to which score (a definition; any fixed bijection
   would do, this one lets one generator call serve the scores one GPU lane
   holds): for slice (b, h) of a batch with H heads, query row i and key j,
   write j = 32 g + 8 q + 4 s + u with s in {0, 1} and q, u in 0..3.  The
   call uses key (seed mod 2^32, seed div 2^32) and counter
   (2 g + s, i, b H + h, offset); its four output words read as 16
   little-endian bytes (byte 4 w + k is bits 8k..8k+7 of word w), and
   u_ij is byte 4 q + u.

``attention_dropout`` follows the forward oracle's steps (scale, mask,
softmax, weighted sum) with the mask applied between the last two.
"""
from __future__ import annotations

import math

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_LOW32 = np.uint64(0xFFFFFFFF)
_SHIFT32 = np.uint64(32)


def philox4x32_10(counter, key):
    """Philox4x32-10.  counter: integer array [..., 4] of 32-bit words, key:
    [..., 2] (broadcast against counter).  Returns uint32 [..., 4]."""
    counter = np.asarray(counter, dtype=np.uint64)
    key = np.asarray(key, dtype=np.uint64)
    c0, c1, c2, c3 = (counter[..., w] for w in range(4))
    k0, k1 = key[..., 0], key[..., 1]
    for _ in range(10):
        prod0 = np.uint64(PHILOX_M0) * c0  # 32 x 32 bits: exact in 64
        prod1 = np.uint64(PHILOX_M1) * c2
        c0, c1, c2, c3 = ((prod1 >> _SHIFT32) ^ c1 ^ k0, prod1 & _LOW32,
                          (prod0 >> _SHIFT32) ^ c3 ^ k1, prod0 & _LOW32)
        k0 = (k0 + np.uint64(PHILOX_W0)) & _LOW32
        k1 = (k1 + np.uint64(PHILOX_W1)) & _LOW32
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def keep_threshold(p_drop) -> int:
    """t = floor(256 (1 - p) + 1/2) for the binary32 drop rate p (reading 2)."""
    p = float(np.float32(p_drop))
    if not (0.0 <= p < 1.0):
        raise ValueError(f"drop rate {p} outside [0, 1)")
    t = math.floor(256.0 * (1.0 - p) + 0.5)
    if t < 1:
        raise ValueError(f"drop rate {p} keeps nothing (t = 0)")
    return t


def dropout_bytes(n_q: int, n_k: int, bh: int, seed: int, offset: int) -> np.ndarray:
    """The bytes u_ij of slice bh (= b H + h), uint8 [n_q, n_k] (reading 4)."""
    n_calls = 2 * ((n_k + 31) // 32)  # counter word c0 runs over 2 g + s
    c0 = np.arange(n_calls, dtype=np.uint64)
    i = np.arange(n_q, dtype=np.uint64)
    ctr = np.zeros((n_q, n_calls, 4), dtype=np.uint64)
    ctr[..., 0] = c0[None, :]
    ctr[..., 1] = i[:, None]
    ctr[..., 2] = bh
    ctr[..., 3] = offset & 0xFFFFFFFF
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    words = philox4x32_10(ctr, key)  # [n_q, n_calls, 4]
    j = np.arange(n_k)
    g, q, s, u = j // 32, (j % 32) // 8, (j % 8) // 4, j % 4
    w = words[:, 2 * g + s, q]  # [n_q, n_k]: word q of call (g, s)
    return ((w >> (8 * u).astype(np.uint32)) & 0xFF).astype(np.uint8)


def attention_dropout_slice(q, k, v, scale: float, causal: bool, p_drop: float,
                            seed: int, offset: int, bh: int):
    """One (batch, head) slice: float64 [N, d] inputs -> (O, lse)."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    n_q, n_k = q.shape[0], k.shape[0]
    s = np.float64(scale) * (q @ k.T)                                       # scale
    if causal:
        s = np.where(np.arange(n_k)[None, :] > np.arange(n_q)[:, None], -np.inf, s)  # mask
    m = s.max(axis=1, initial=-np.inf)                                      # softmax
    seen = np.isfinite(m)
    p = np.zeros_like(s)
    p[seen] = np.exp(s[seen] - m[seen][:, None])
    l = p.sum(axis=1)
    p[seen] /= l[seen][:, None]
    lse = np.full(n_q, -np.inf)
    lse[seen] = m[seen] + np.log(l[seen])
    t = keep_threshold(p_drop)                                              # dropout
    keep = dropout_bytes(n_q, n_k, bh, seed, offset) < t
    o = ((p * keep) @ v) * (256.0 / t)                                      # weighted sum
    return o, lse


def attention_dropout(q, k, v, scale: float, causal: bool, p_drop: float, seed: int,
                      offset: int, slices=None):
    """[B, H, N, d] float64 inputs -> (O [B, H, N, d], lse [B, H, N]).

    With ``slices`` (a list of (b, h)), only those slices are computed; the
    others are left NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, N, d = q.shape
    o = np.full((B, H, N, v.shape[-1]), np.nan)
    lse = np.full((B, H, N), np.nan)
    todo = slices if slices is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        o[b, h], lse[b, h] = attention_dropout_slice(q[b, h], k[b, h], v[b, h], scale, causal,
                                                     p_drop, seed, offset, b * H + h)
    return o, lse
