"""Packed ternary-weight GEMV / GEMM for AMD Instinct MI355X (gfx950).

The product lives in ``libtq.so`` (HIP kernels behind the C ABI of
``include/tq.h``); ``ternary_weight_amd.tq`` is its thin Python binding.
Importing the package loads nothing; the first call into ``tq`` loads the
library and fails loudly if it has not been built.
"""
from . import tq  # noqa: F401

__all__ = ["tq"]
