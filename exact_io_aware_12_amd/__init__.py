"""Fused exact attention for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libfa355.so`` (hand-written HIP
kernels); ``exact_io_aware_12_amd.fa`` is its thin ctypes binding. Importing
this package loads nothing; the library is opened on first use.
"""
__all__ = ["fa", "inputs"]
