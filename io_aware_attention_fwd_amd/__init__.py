"""MI355X (gfx950) FlashAttention forward: Python side of the C-ABI library.

``fa_fwd`` / ``fa_fwd_fp8`` / ``fa_fwd_varlen`` / ``fa_fwd_dropout`` /
``fa_bwd`` / ``fa_qkv_proj`` mirror the C entry points in ``include/fa.h`` and
only marshal arguments; ``fwd``, ``fwd_varlen``, ``fwd_dropout``, ``bwd`` and
``qkv_proj`` are convenience wrappers that allocate the outputs with torch and call them.  The
shared library is loaded on first use and a missing or unloadable library
raises -- there is no fallback path.
"""
from ._lib import (  # noqa: F401
    FA_DTYPE_F16,
    FA_DTYPE_BF16,
    FA_DTYPE_FP8_E4M3,
    FaError,
    bwd,
    fa_bwd,
    fa_fwd,
    fa_fwd_dropout,
    fa_fwd_fp8,
    fa_fwd_varlen,
    fa_qkv_proj,
    fa_strerror,
    fa_version,
    fwd,
    fwd_dropout,
    fwd_varlen,
    library_path,
    load,
    qkv_proj,
)
