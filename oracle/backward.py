"""Gradients of the attention forward pass in float64 (the backward pass).

Given the forward definition of ``oracle.attention`` for one (batch, head)
slice -- S = scale * Q K^T, causal mask, P = softmax of each row, O = P V --
and the gradient dO of a scalar loss with respect to O, the chain rule gives

1. dV = P^T dO
2. dP = dO V^T
3. dS_ij = P_ij * (dP_ij - sum_k P_ik dP_ik)      (softmax Jacobian, row by row)
4. dQ = scale * dS K
5. dK = scale * dS^T Q

Masked entries have P_ij = 0 and so dS_ij = 0.  The row term
sum_k P_ik dP_ik equals sum_c dO_ic O_ic, which is how a tiled backward pass
computes it without the matrix.

Passages: the backward pass is what recomputation ("0 MB (重计算)" in the Flash
Attention 2 memory table of page "Optimization Flash Attention 基准测试") is
for -- P is rebuilt from Q, K and the saved logsumexp instead of being stored
-- and the training/inference section promised by that page's table of
contents.  The formulas themselves are not on the pages: they are the
derivative of the definition above, written out here in the plainest form
(the whole P of a slice is materialised).
"""
from __future__ import annotations

import numpy as np


def _probabilities(q, k, scale, causal):
    s = np.float64(scale) * (q @ k.T)
    if causal:
        n_q, n_k = s.shape
        s = np.where(np.arange(n_k)[None, :] > np.arange(n_q)[:, None], -np.inf, s)
    m = s.max(axis=1, initial=-np.inf)
    p = np.zeros_like(s)
    seen = np.isfinite(m)
    p[seen] = np.exp(s[seen] - m[seen][:, None])
    l = p.sum(axis=1)
    p[seen] /= l[seen][:, None]
    return p


def attention_backward_slice(q, k, v, do, scale: float, causal: bool):
    """One (batch, head) slice: float64 [N, d] inputs and dO -> (dQ, dK, dV)."""
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    p = _probabilities(q, k, scale, causal)
    dv = p.T @ do                                            # 1
    dp = do @ v.T                                            # 2
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))     # 3
    dq = np.float64(scale) * (ds @ k)                        # 4
    dk = np.float64(scale) * (ds.T @ q)                      # 5
    return dq, dk, dv


def attention_backward(q, k, v, do, scale: float, causal: bool, slices=None):
    """[B, H, N, d] float64 inputs and dO -> (dQ, dK, dV), each [B, H, N, d].

    With ``slices`` (a list of (b, h)), only those slices are computed; the
    others are left NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, N, d = q.shape
    out = [np.full((B, H, N, d), np.nan, dtype=np.float64) for _ in range(3)]
    todo = slices if slices is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        g = attention_backward_slice(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal)
        for dst, val in zip(out, g):
            dst[b, h] = val
    return tuple(out)
