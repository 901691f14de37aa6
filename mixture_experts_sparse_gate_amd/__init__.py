"""Sparse-gated Mixture-of-Experts layer forward for MI355X (gfx950).

The HIP kernels live in ``csrc/`` and are compiled into ``libmoe_gfx950.so``
behind the C ABI declared in ``include/moe.h``; ``api`` is a thin ctypes
binding over it. Importing this package does not load the library: ``api``
loads it on first use and raises if it is missing.
"""
