"""MI355X (gfx950) FlashAttention forward: Python side of the C-ABI library.

``fa_fwd`` / ``fa_fwd_fp8`` mirror the C entry points in ``include/fa.h`` and
only marshal arguments; ``fwd`` is a convenience wrapper that allocates the
outputs with torch and calls ``fa_fwd``.  The shared library is loaded on first
use and a missing or unloadable library raises -- there is no fallback path.
"""
from ._lib import (  # noqa: F401
    FA_DTYPE_F16,
    FA_DTYPE_BF16,
    FA_DTYPE_FP8_E4M3,
    FaError,
    fa_fwd,
    fa_fwd_fp8,
    fa_strerror,
    fa_version,
    fwd,
    library_path,
    load,
)
