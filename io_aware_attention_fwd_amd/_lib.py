"""ctypes binding of libfa.so: argument marshalling only.

``fa_fwd``, ``fa_fwd_fp8``, ``fa_fwd_varlen``, ``fa_fwd_dropout``, ``fa_bwd``,
``fa_bwd_noalloc``, ``fa_qkv_proj``, ``fa_fwd_tile``, ``fa_strerror`` and ``fa_version`` take the same arguments as
the C functions declared in ``include/fa.h`` (device pointers as Python ints,
the stream as a ``hipStream_t`` int or None).  ``fwd``, ``fwd_varlen``,
``fwd_dropout``, ``bwd`` and ``qkv_proj`` allocate
their outputs (and the backward workspace) with torch on the inputs' device
and call the library on torch's current stream.  Every step of the computation runs
in the library's HIP kernels; if the library is missing or fails to load, the
call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # imported first: libfa.so then binds to the HIP runtime torch loaded

FA_DTYPE_F16 = 0
FA_DTYPE_BF16 = 1
FA_DTYPE_FP8_E4M3 = 2

_LIB = None
_HERE = os.path.dirname(os.path.abspath(__file__))


class FaError(RuntimeError):
    """A nonzero return code from libfa.so."""

    def __init__(self, code: int, where: str = "fa_fwd"):
        self.code = code
        super().__init__(f"{where} returned {code}: {fa_strerror(code) if _LIB else 'library not loaded'}")


def library_path() -> str:
    """The in-tree libfa.so, or the build named by the FA_LIBRARY environment
    variable (used to run the CPU ABI tests against an instrumented host build)."""
    return os.environ.get("FA_LIBRARY") or os.path.join(_HERE, "libfa.so")


def load() -> ctypes.CDLL:
    """Load libfa.so once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        _LIB = open_library(library_path())
    return _LIB


def open_library(path: str) -> ctypes.CDLL:
    """A handle on one build of the library (libfa.so, or libfa_sync.so with its
    extra barriers) with every entry point's argument types set."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, cf, ci, ci, vp]
    lib.fa_fwd.restype = ci
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, cf, ci, cf, cf, cf, vp]
    lib.fa_fwd_fp8.restype = ci
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, ci, vp]
    lib.fa_fwd_varlen.restype = ci
    lib.fa_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, cf, ci, ci, cf, ctypes.c_ulonglong,
                                   ctypes.c_uint, vp]
    lib.fa_fwd_dropout.restype = ci
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, cf, ci, ci, vp]
    lib.fa_bwd.restype = ci
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, cf, ci, ci, vp]
    lib.fa_bwd_noalloc.restype = ci
    lib.fa_qkv_proj.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, vp]
    lib.fa_qkv_proj.restype = ci
    lib.fa_fwd_tile.argtypes = [ci, ci, ci, ci, ci, ctypes.POINTER(ctypes.c_int)]
    lib.fa_fwd_tile.restype = ci
    lib.fa_strerror.argtypes = [ci]
    lib.fa_strerror.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ci
    return lib


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream) -> int:
    return load().fa_fwd(q, k, v, o, lse, B, H, N, d, scale, int(causal), dtype, stream)


def fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, scale, causal, q_descale, k_descale, v_descale, stream) -> int:
    return load().fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, scale, int(causal), q_descale, k_descale, v_descale, stream)


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, H, total, max_seqlen, d, scale, causal, dtype, stream) -> int:
    return load().fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, H, total, max_seqlen, d, scale, int(causal), dtype,
                                stream)


def fa_fwd_dropout(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, p_drop, seed, offset, stream) -> int:
    return load().fa_fwd_dropout(q, k, v, o, lse, B, H, N, d, scale, int(causal), dtype, p_drop, seed, offset, stream)


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, dtype, stream) -> int:
    return load().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, int(causal), dtype, stream)


def fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, dtype, stream) -> int:
    return load().fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, int(causal), dtype, stream)


def fa_qkv_proj(x, w, bias, q, k, v, B, N, D, H, d, dtype, stream) -> int:
    return load().fa_qkv_proj(x, w, bias, q, k, v, B, N, D, H, d, dtype, stream)


FA_TILE_DENSE = 0
FA_TILE_VARLEN = 1
FA_TILE_DROPOUT = 2


def fa_fwd_tile(N, d, causal, dtype, mode, tile) -> int:
    return load().fa_fwd_tile(N, d, int(causal), dtype, mode, tile)


def fwd_tile(N: int, d: int, causal: bool, dtype: int, mode: int = FA_TILE_DENSE) -> str:
    """The kernel shape a forward call runs, as the FA_TILE string QWxNWxBCxSCHEDxWPE."""
    t = (ctypes.c_int * 5)()
    rc = fa_fwd_tile(N, d, causal, dtype, mode, t)
    if rc != 0:
        raise FaError(rc, "fa_fwd_tile")
    return "x".join(str(x) for x in t)


def fa_strerror(code: int) -> str:
    return load().fa_strerror(code).decode()


def fa_version() -> int:
    return load().fa_version()


_TORCH_DTYPES = {torch.float16: FA_DTYPE_F16, torch.bfloat16: FA_DTYPE_BF16, torch.float8_e4m3fn: FA_DTYPE_FP8_E4M3}


def _require(t: torch.Tensor, name: str, shape=None, dtype=None) -> None:
    """Shape, dtype and contiguity of one tensor argument (before any device check)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(ref: torch.Tensor, stream, **tensors) -> None:
    """Every tensor (and the stream, if given) on the GPU that holds ``ref``.

    Runs after the shape checks and before the library call: the kernels take
    raw device pointers, so a host tensor or one on another GPU would make
    them read or write memory that is not the tensor's.
    """
    if ref.device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {ref.device}")
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, not on {ref.device} with the other inputs")
    if stream is not None and getattr(stream, "device", ref.device) != ref.device:
        raise ValueError(f"stream belongs to {stream.device}, not to {ref.device}")


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float, causal: bool = False, *,
        descale=(1.0, 1.0, 1.0), out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
        stream: torch.cuda.Stream | None = None):
    """Attention forward on [B, H, N, d] device tensors; returns (O, lse).

    fp8 inputs are ``torch.float8_e4m3fn`` (or uint8 codes) with per-tensor
    ``descale = (q, k, v)``; their O is bfloat16.
    """
    if q.dtype == torch.uint8:
        q, k, v = (t.view(torch.float8_e4m3fn) for t in (q, k, v))
    if q.dtype not in _TORCH_DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError(f"unsupported dtypes {q.dtype}, {k.dtype}, {v.dtype}")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q, k, v must share one [B, H, N, d] shape, got {tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, N, d = q.shape
    dt = _TORCH_DTYPES[q.dtype]
    o_dtype = torch.bfloat16 if dt == FA_DTYPE_FP8_E4M3 else q.dtype
    if out is not None:
        _require(out, "out", (B, H, N, d), o_dtype)
    if lse is not None:
        _require(lse, "lse", (B, H, N), torch.float32)
    _same_device(q, stream, k=k, v=v, out=out, lse=lse)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=o_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    s = stream.cuda_stream
    if dt == FA_DTYPE_FP8_E4M3:
        rc = fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                        B, H, N, d, float(scale), causal, float(descale[0]), float(descale[1]), float(descale[2]), s)
    else:
        rc = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    B, H, N, d, float(scale), causal, dt, s)
    if rc != 0:
        raise FaError(rc)
    return out, lse


def fwd_dropout(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float, causal: bool, p_drop: float,
                seed: int, offset: int = 0, *, stream: torch.cuda.Stream | None = None):
    """Attention forward with dropout on [B, H, N, d] binary16/bfloat16 device
    tensors; returns (O, lse).  The mask is a function of (seed, offset) and
    the score's position (see ``fa_fwd_dropout`` in include/fa.h)."""
    if q.dtype not in (torch.float16, torch.bfloat16) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError(f"unsupported dtypes {q.dtype}, {k.dtype}, {v.dtype}")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q, k, v must share one [B, H, N, d] shape, got {tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, N, d = q.shape
    _same_device(q, stream, k=k, v=v)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    rc = fa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
                        float(scale), causal, _TORCH_DTYPES[q.dtype], float(p_drop), int(seed), int(offset),
                        stream.cuda_stream)
    if rc != 0:
        raise FaError(rc, "fa_fwd_dropout")
    return out, lse


def fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
               scale: float, causal: bool = False, *, out: torch.Tensor | None = None,
               lse: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None):
    """Attention forward on packed [total, H, d] sequences; returns (O [total, H, d], lse [H, total]).

    ``cu_seqlens`` is an int32 device tensor of B+1 row offsets.  fp8 inputs
    (``torch.float8_e4m3fn`` or uint8 codes) are taken with descales of 1.
    """
    if q.dtype == torch.uint8:
        q, k, v = (t.view(torch.float8_e4m3fn) for t in (q, k, v))
    if q.dtype not in _TORCH_DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError(f"unsupported dtypes {q.dtype}, {k.dtype}, {v.dtype}")
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q, k, v must share one [total, H, d] shape, got {tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise TypeError("cu_seqlens must be a contiguous 1-D int32 tensor")
    total, H, d = q.shape
    B = cu_seqlens.numel() - 1
    dt = _TORCH_DTYPES[q.dtype]
    o_dtype = torch.bfloat16 if dt == FA_DTYPE_FP8_E4M3 else q.dtype
    if out is not None:
        _require(out, "out", (total, H, d), o_dtype)
    if lse is not None:
        _require(lse, "lse", (H, total), torch.float32)
    _same_device(q, stream, k=k, v=v, cu_seqlens=cu_seqlens, out=out, lse=lse)
    if out is None:
        out = torch.empty((total, H, d), dtype=o_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    rc = fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), cu_seqlens.data_ptr(),
                       B, H, total, int(max_seqlen), d, float(scale), causal, dt, stream.cuda_stream)
    if rc != 0:
        raise FaError(rc, "fa_fwd_varlen")
    return out, lse


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
        scale: float, causal: bool = False, *, stream: torch.cuda.Stream | None = None):
    """Gradients of ``fwd`` on [B, H, N, d] f16/bf16 device tensors; returns (dQ, dK, dV)."""
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError(f"the backward pass takes float16 or bfloat16, got {q.dtype}")
    for t in (k, v, o, dout):
        if t.dtype != q.dtype or t.shape != q.shape or not t.is_contiguous():
            raise ValueError("q, k, v, o, dout must share one contiguous [B, H, N, d] shape and dtype")
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, H, N, d] tensor")
    B, H, N, d = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    _same_device(q, stream, k=k, v=v, o=o, lse=lse, dout=dout)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    rc = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, N, d, float(scale), causal, _TORCH_DTYPES[q.dtype],
                stream.cuda_stream)
    if rc != 0:
        raise FaError(rc, "fa_bwd")
    return dq, dk, dv


def qkv_proj(x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor | None, H: int, d: int, *,
             stream: torch.cuda.Stream | None = None):
    """Fused QKV projection: x [B, N, D], w [3 H d, D], bias [3 H d] or None
    (binary16 or bfloat16 device tensors); returns (Q, K, V), each [B, H, N, d]."""
    if x.dtype not in (torch.float16, torch.bfloat16) or w.dtype != x.dtype or (bias is not None and bias.dtype != x.dtype):
        raise TypeError("x, w and bias must share one 16-bit dtype")
    if x.dim() != 3 or w.shape != (3 * H * d, x.shape[2]) or (bias is not None and bias.shape != (3 * H * d,)):
        raise ValueError(f"shapes x {tuple(x.shape)}, w {tuple(w.shape)} do not match H={H}, d={d}")
    if not (x.is_contiguous() and w.is_contiguous() and (bias is None or bias.is_contiguous())):
        raise ValueError("x, w and bias must be contiguous")
    B, N, D = x.shape
    _same_device(x, stream, w=w, bias=bias)
    q, k, v = (torch.empty((B, H, N, d), dtype=x.dtype, device=x.device) for _ in range(3))
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    rc = fa_qkv_proj(x.data_ptr(), w.data_ptr(), None if bias is None else bias.data_ptr(), q.data_ptr(),
                     k.data_ptr(), v.data_ptr(), B, N, D, H, d, _TORCH_DTYPES[x.dtype], stream.cuda_stream)
    if rc != 0:
        raise FaError(rc, "fa_qkv_proj")
    return q, k, v
