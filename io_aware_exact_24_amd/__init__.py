"""Exact, IO-aware attention (forward + recompute backward) for MI355X / gfx950.

The compute lives in libfa.so (hand-written HIP kernels behind the C ABI in
include/fa.h).  This package is a thin ctypes binding with the same entry-point
names; it loads the library on first use and raises if it is missing.
"""

from .binding import (  # noqa: F401
    FA_BF16,
    FA_F32,
    FaError,
    fa_bwd,
    fa_bwd_workspace_size,
    fa_fwd,
    fa_status_string,
    library_path,
    load_library,
    forward,
    backward,
)
