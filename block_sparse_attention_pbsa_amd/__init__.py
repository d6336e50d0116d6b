"""PBSA on MI355X: Persistent Block-Sparse Attention as a C-ABI library of gfx950 HIP kernels.

Importing the package loads nothing.  ``ops`` loads ``libpbsa.so`` on first use and
raises if it is missing; there is no fallback path.
"""
__all__ = ["synth", "ops", "runtime"]
