"""Packed quantized linear layers on MI355X (gfx950): W4 group quantization,
SpQR (3-bit bi-level + CSR fp16 outliers) and SmoothQuant W8A8.

The compute lives in libqlin.so (hand-written HIP kernels behind the C ABI of
include/qlin.h); ``qlin`` is its ctypes binding.  Importing the binding fails
loudly when the library has not been built.
"""
__all__ = ["qlin"]
