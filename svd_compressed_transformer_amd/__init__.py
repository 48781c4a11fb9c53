"""Fused low-rank (SVD-compressed) transformer-layer hot path for AMD Instinct MI355X (gfx950).

``fsvd`` is the ctypes binding of the HIP library ``libfsvd.so`` (C ABI in ``include/fsvd.h``);
``inputs`` holds the seeded synthetic input generators.  Importing the package loads nothing.
"""
__all__ = ["fsvd", "inputs"]
