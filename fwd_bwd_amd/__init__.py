"""fwd_bwd_amd: fused neighborhood attention forward/backward for MI355X (gfx950).

The computation runs in libna.so (HIP kernels behind the C ABI of include/na.h);
``fwd_bwd_amd.na`` is a thin ctypes binding with the same entry-point names.
"""
from .na import (  # noqa: F401
    NaError, na_bwd, na_fwd, neighborhood_attention, window_start, inverse_window,
)

__all__ = ["na_fwd", "na_bwd", "neighborhood_attention", "window_start", "inverse_window",
           "NaError"]
