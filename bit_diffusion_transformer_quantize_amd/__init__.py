"""SVDQuant W4A4 quantized linear layer for AMD Instinct MI355X (gfx950).

The compute lives in ``libsvdq.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/svdq.h``); ``svdq`` is its ctypes binding.
"""
from . import svdq  # noqa: F401

__version__ = "0.1.0"
