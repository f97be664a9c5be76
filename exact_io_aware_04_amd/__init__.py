"""MI355X (gfx950) fused exact attention: forward and recomputing backward.

The compute path is the HIP library libfa.so (C ABI in include/fa.h); the
Python side only marshals arguments. Import `exact_io_aware_04_amd.fa` to load
the library; importing the package itself loads nothing.
"""
__all__ = ["fa"]
