"""Fused exact attention for one AMD Instinct MI355X (gfx950).

The compute lives in a C-ABI shared library (``include/attn.h``) built from
``csrc/``; ``io_aware_exact_06_amd.attn`` is the thin ctypes binding over it.
Importing this package loads nothing: the library is opened on first use and
a missing library is an error, never a fallback.
"""
__all__ = ["attn", "inputs"]
