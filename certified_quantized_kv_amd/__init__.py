"""Certified quantized-KV decode attention on MI355X (HIP, gfx950).

Thin ctypes binding over the C ABI in ``include/ckv.h``: argument marshalling
only.  Every step of the decode path runs in the HIP kernels of
``libckv.so``; there is no Python or CPU fallback.  PyTorch is used only for
device memory and the current stream.
"""
from .binding import (  # noqa: F401
    REPORT_DTYPE,
    Cache,
    CkvError,
    Thresholds,
    default_thresholds,
    lib,
)
