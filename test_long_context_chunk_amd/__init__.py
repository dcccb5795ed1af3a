"""Chunk-wise test-time-training (TTT) inner loop for MI355X (gfx950).

The computation lives in a HIP shared library with a C ABI (include/ttt.h); this package
is its thin Python binding plus the build script.
"""
from ._binding import (ABI_VERSION, SIGNATURES, STATUS, TTT, TTTError, gemm_pair_test_hook, gemm_test_hook,
                       grad_test_hook, load_library, to_device)
from .build import lib_path

__all__ = ["ABI_VERSION", "SIGNATURES", "STATUS", "TTT", "TTTError", "gemm_pair_test_hook", "gemm_test_hook",
           "grad_test_hook",
           "load_library", "to_device", "lib_path"]
