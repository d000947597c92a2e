"""Exact, IO-aware attention (FlashAttention-2 style) for AMD MI355X.

The computation lives in hand-written gfx950 HIP kernels behind the C ABI
of ``libfa.so`` (declared in ``include/fa.h``). ``_lib`` is the ctypes
binding with the C names; ``attention`` allocates torch tensors and calls
it. Importing this package does not load the library; the first call does,
and fails loudly if it has not been built.
"""
from . import _lib  # noqa: F401

__all__ = ["_lib"]
