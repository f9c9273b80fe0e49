"""MI355X-native FP4 block-scaled quantizer and GEMM (``libfp4q``).

The compute path is the C-ABI library ``libfp4q.so`` (hand-written HIP for
gfx950) declared in ``include/fp4q.h``; ``binding`` is a thin ctypes layer over
it with the same entry-point names.  Importing this package does not touch the
GPU; the binding loads the library on first use and raises if it is missing.
"""
__all__ = ["binding", "synth"]
