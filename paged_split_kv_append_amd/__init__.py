"""Paged split-KV attention for AMD Instinct MI355X (gfx950).

The product is the C-ABI library ``libnbx_paged.so`` built from ``csrc/``
(HIP kernels + host entry points declared in ``include/nbx_paged.h``).
``binding`` is a thin ctypes layer with the same entry-point names; it loads
the library on first use and raises if it is missing.  ``synth`` draws seeded
inputs.
"""
__all__ = ["binding", "synth"]
