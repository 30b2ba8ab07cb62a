"""MI355X (gfx950) top-k selection and top-K sparse-attention decode.

The work runs in the HIP library ``libatopk.so`` (C ABI, header
``include/atopk.h``); this package is a thin ctypes binding over it.
"""
