"""Block-quantized weight dequantize-and-multiply (Q8_0, Q4_K, Q6_K, INT4 group-128) for gfx950.

The product is libqmv.so (C ABI in include/qmv.h, HIP kernels in csrc/); the
``qmv`` module is its Python binding.  Importing this package loads nothing;
the library is loaded on the first call into ``qmv``.
"""
from . import qmv  # noqa: F401

__all__ = ["qmv"]
