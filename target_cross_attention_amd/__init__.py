"""MI355X-native Stacked Target Cross Attention (STCA) forward pass.

The compute lives in ``libstca.so`` (HIP kernels for gfx950 behind the C ABI of
``include/stca.h``); ``binding`` is a thin ctypes layer with the same call names.
Importing ``binding`` fails loudly when the library has not been built.
"""
__all__ = ["binding", "build"]
