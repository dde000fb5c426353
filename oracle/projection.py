"""The fused QKV projection in float64: the step before attention.

Test infrastructure only (see the package docstring).

Passage: page "FlashAttention与TensorRT 10集成", section "算子融合的极致优化",
item 1, merges the input projection with the transpose and rearrangement
that turn its result into the attention inputs.  The page gives no formula.
Reading (the usual multi-head attention input projection):

* X is the layer input, token-major [B, N, D] (D = model width).
* W is one packed weight [3 H d, D] for the three projections, stored
  [out, in] like a linear layer's weight, with an optional bias [3 H d]:
      Y = X W^T + bias          ([B, N, 3 H d])
* Output feature f = s H d + h d + c belongs to tensor s (0 = Q, 1 = K,
  2 = V), head h, column c: the transpose and rearrangement place it at
      out_s[b, h, n, c] = Y[b, n, s H d + h d + c],
  the dense [B, H, N, d] layout the attention kernels read.

The matrix product is numpy's float64 ``@`` (a library primitive); the
layout change is a reshape and a transpose.
"""
from __future__ import annotations

import numpy as np


def qkv_projection(x, w, bias, H: int, d: int):
    """x: [B, N, D], w: [3 H d, D], bias: [3 H d] or None (all float64).
    Returns (Q, K, V), each float64 [B, H, N, d]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, N, D = x.shape
    assert w.shape == (3 * H * d, D), (w.shape, (3 * H * d, D))
    y = x @ w.T                                     # projection
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, None, :]
    y = y.reshape(B, N, 3, H, d).transpose(2, 0, 3, 1, 4)  # rearrange: [3, B, H, N, d]
    return y[0], y[1], y[2]
