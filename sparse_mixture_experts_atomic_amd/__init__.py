"""Sparse Mixture-of-Experts FFN layer forward for AMD MI355X (gfx950).

The compute lives in libmoe.so (hand-written HIP kernels behind a C ABI,
declared in include/moe.h).  ``_lib`` is the ctypes binding, ``layer`` a
buffer-owning runner of the five calls.
"""
from . import _lib
from ._lib import MoEError, lib
from .layer import MoELayer

__all__ = ["_lib", "MoEError", "lib", "MoELayer"]
