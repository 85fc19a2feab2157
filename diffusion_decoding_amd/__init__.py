"""Block-diffusion denoise path for MI355X (gfx950).

The computation lives in libdg.so (HIP kernels behind the C ABI of
include/dg.h); this package is its binding.  Importing it does not load the
library; the first call does, and fails loudly if it has not been built.
"""
from . import _lib
from ._lib import DGError, ENTRY_POINTS, LIB_PATH, load

__all__ = ["DGError", "ENTRY_POINTS", "LIB_PATH", "load"]
