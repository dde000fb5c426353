"""Attention forward in float64: the definition the GPU kernels must reach.

What is computed, per (batch, head) slice with Q, K, V of shape [N, d]:

1. scores  S = scale * Q K^T                      (N x N, materialised)
2. mask    S_ij = -inf for j > i when causal      (diagonal kept)
3. softmax m_i = max_j S_ij, P_ij = exp(S_ij - m_i), l_i = sum_j P_ij
4. output  O_i = sum_j (P_ij / l_i) V_j
5. lse_i = m_i + ln(l_i)  (natural log, scale included)

Passages followed:

* Steps 1-4 in this order are the fused sequence "scale, mask, softmax,
  weighted sum" of page "FlashAttention与TensorRT 10集成", section
  "算子融合的极致优化" (operator fusion), item 2.
* Materialising the whole N x N matrix is what that page's section "技术痛点"
  calls the standard implementation; FlashAttention reaches the same result
  exactly (up to rounding order) without storing it, so this plain definition
  is the oracle, not the tiled algorithm.
* ``causal`` is the flag of the tuning dict on page "从RTX 3090到H100：
  FlashAttention在NVIDIA各代GPU架构上的性能全景分析", section 3.2.  The pages do
  not say how the mask is aligned; the reading taken is the lower triangle with
  the diagonal kept (query i may see keys j <= i), which for equal query and
  key lengths is the only natural one.
* Step 5, the per-row logsumexp, is not on the pages.  It is what a backward
  pass needs to recompute P instead of storing it ("0 MB (重计算)" in the
  Flash Attention 2 memory table of page "Optimization Flash Attention
  基准测试").  Reading: natural logarithm of sum_j exp(S_ij) over the keys the
  row may see, with the scale included.
* A row with no visible key (impossible for causal self-attention with equal
  lengths, kept for completeness) gives O_i = 0 and lse_i = -inf.

The score matrix is built ``row_chunk`` query rows at a time only to bound
memory; each chunk is the plain definition above.

``attention_varlen`` applies the same definition to sequences of different
lengths packed back to back ([total, H, d], sequence b owning rows
cu[b]..cu[b+1]-1): every (sequence, head) is its own attention problem, and
a causal row sees the keys of its own sequence up to itself.  The pages pad
unaligned lengths (page "从RTX 3090到H100：FlashAttention在NVIDIA各代GPU架构上
的性能全景分析", section 3.2, common pitfalls item 2) and name dynamic shapes as
a direction (page "FlashAttention与TensorRT 10集成", section "推理优化的未来方
向" item 1); computing each sequence on its own rows is what padding with
masked keys would give for the rows that exist.
"""
from __future__ import annotations

import numpy as np


def attention_slice(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                    causal: bool, row_chunk: int = 1024):
    """One (batch, head) slice.  q, k, v: float64 [N, d].  Returns (O, lse)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, d = q.shape
    n_k = k.shape[0]
    o = np.zeros((n_q, v.shape[1]), dtype=np.float64)
    lse = np.full(n_q, -np.inf, dtype=np.float64)
    keys = np.arange(n_k)[None, :]
    for r0 in range(0, n_q, row_chunk):
        r1 = min(n_q, r0 + row_chunk)
        s = np.float64(scale) * (q[r0:r1] @ k.T)                  # 1. scale
        if causal:                                                 # 2. mask
            rows = np.arange(r0, r1)[:, None]
            s = np.where(keys > rows, -np.inf, s)
        m = s.max(axis=1, initial=-np.inf)                         # 3. softmax
        seen = np.isfinite(m)
        p = np.exp(s[seen] - m[seen][:, None])
        l = p.sum(axis=1)
        o[r0:r1][seen] = (p / l[:, None]) @ v                      # 4. weighted sum
        lse[r0:r1][seen] = m[seen] + np.log(l)                     # 5. logsumexp
    return o, lse


def slice_sample(B: int, H: int, count: int = 8, seed: int = 1234):
    """The (b, h) slices checked on large shapes.

    (0, 0), (B-1, H-1), then ``count - 2`` more drawn without replacement from
    the remaining flat indices by ``numpy.random.default_rng(seed).choice``.
    Small shapes (B*H <= count) use every slice.
    """
    total = B * H
    if total <= count:
        return [(i // H, i % H) for i in range(total)]
    first, last = 0, total - 1
    rest = np.array([i for i in range(total) if i not in (first, last)])
    pick = np.random.default_rng(seed).choice(rest, count - 2, replace=False)
    flat = [first, last] + sorted(int(x) for x in pick)
    return [(i // H, i % H) for i in flat]


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool,
              slices=None, row_chunk: int = 1024):
    """[B, H, N, d] float64 inputs -> (O [B,H,N,d], lse [B,H,N]) in float64.

    With ``slices`` (a list of (b, h)), only those slices are computed; the
    others are left NaN so that an accidental comparison against them fails.
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, N, d = q.shape
    o = np.full((B, H, N, v.shape[-1]), np.nan, dtype=np.float64)
    lse = np.full((B, H, N), np.nan, dtype=np.float64)
    todo = slices if slices is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        o[b, h], lse[b, h] = attention_slice(q[b, h], k[b, h], v[b, h], scale, causal, row_chunk)
    return o, lse


def attention_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu, scale: float, causal: bool,
                     sequences=None, row_chunk: int = 1024):
    """Packed [total, H, d] float64 inputs and B+1 offsets ``cu`` -> (O [total,H,d], lse [H,total]).

    With ``sequences`` (a list of sequence indices), only those are computed;
    the rows of the others stay NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    total, H, d = q.shape
    cu = [int(x) for x in cu]
    o = np.full((total, H, v.shape[-1]), np.nan, dtype=np.float64)
    lse = np.full((H, total), np.nan, dtype=np.float64)
    todo = sequences if sequences is not None else range(len(cu) - 1)
    for b in todo:
        r0, r1 = cu[b], cu[b + 1]
        for h in range(H):
            o[r0:r1, h], lse[h, r0:r1] = attention_slice(q[r0:r1, h], k[r0:r1, h], v[r0:r1, h], scale, causal,
                                                         row_chunk)
    return o, lse
