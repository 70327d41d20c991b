"""Additive multi-codebook (AQLM) quantized linear layers on MI355X (gfx950).

The compute path is the HIP library libaqlm_mi355x.so (C ABI in
include/aqlm.h); `AqlmLayer` is its thin torch-facing binding. Importing the
package does not load the library; the first call does, and fails loudly if
it has not been built.
"""
from ._lib import (AqlmError, AqlmLayer, gemv_batched, library_path, load_library,  # noqa: F401
                   status_string)

__all__ = ["AqlmLayer", "AqlmError", "gemv_batched", "load_library", "library_path",
           "status_string"]
