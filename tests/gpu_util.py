"""Helpers shared by the GPU tests: device upload, library call, oracle comparison."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from io_aware_attention_fwd_amd import _lib, gen

# Tolerances: max |O_gpu - O_ref| per storage format; lse relative to max(1, |lse|).
O_TOL = {"f16": 1e-2, "bf16": 2e-2, "fp8": 6e-2}
LSE_TOL = 1e-3

_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


def to_device(x: gen.Inputs, device="cuda"):
    def t(a):
        if x.dtype == "f16":
            return torch.from_numpy(a).to(device)
        if x.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(a).view(torch.float8_e4m3fn).to(device)

    return t(x.q), t(x.k), t(x.v)


def run_gpu(x: gen.Inputs, scale: float, causal: bool, stream=None):
    q, k, v = to_device(x)
    ds = (x.descale["q"], x.descale["k"], x.descale["v"])
    o, lse = _lib.fwd(q, k, v, scale, causal, descale=ds, stream=stream)
    torch.cuda.synchronize()
    return o, lse


def o_to_numpy(o: torch.Tensor) -> np.ndarray:
    return o.float().cpu().numpy().astype(np.float64)


def dequant(x: gen.Inputs, b=None, h=None):
    sl = (slice(None),) * 2 if b is None else (b, h)
    return (oracle.dequantize(x.q[sl], x.dtype, x.descale["q"]),
            oracle.dequantize(x.k[sl], x.dtype, x.descale["k"]),
            oracle.dequantize(x.v[sl], x.dtype, x.descale["v"]))


def compare(x: gen.Inputs, o_gpu: np.ndarray, lse_gpu: np.ndarray, scale: float, causal: bool, slices=None,
            o_tol=None):
    """Oracle on the given (b, h) slices (all when None) against the GPU outputs.

    Returns (max |dO|, max relative dlse, max |O_ref|) and asserts the bars.
    """
    B, H, N, d = x.shape
    if slices is None:
        slices = [(b, h) for b in range(B) for h in range(H)]
    tol = O_TOL[x.dtype] if o_tol is None else o_tol
    worst_o = worst_l = ref_mag = 0.0
    for b, h in slices:
        q, k, v = dequant(x, b, h)
        o_ref, lse_ref = oracle.attention_slice(q, k, v, scale, causal)
        do = np.abs(o_gpu[b, h] - o_ref).max()
        dl = (np.abs(lse_gpu[b, h] - lse_ref) / np.maximum(1.0, np.abs(lse_ref))).max()
        assert np.isfinite(o_gpu[b, h]).all() and np.isfinite(lse_gpu[b, h]).all(), (b, h)
        assert do <= tol, f"slice {(b, h)}: max|dO| = {do:.3g} > {tol}"
        assert dl <= LSE_TOL, f"slice {(b, h)}: max rel dlse = {dl:.3g} > {LSE_TOL}"
        worst_o, worst_l = max(worst_o, do), max(worst_l, dl)
        ref_mag = max(ref_mag, np.abs(o_ref).max())
    return worst_o, worst_l, ref_mag
