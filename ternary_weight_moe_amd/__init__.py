"""Routed ternary-weight MoE FFN for MI355X (gfx950).

The compute lives in libmaple_moe.so (hand-written HIP kernels behind the C ABI
of include/maple_moe.h); ``_native`` is its ctypes binding and ``synth`` the
seeded synthetic-input generator.
"""
from . import _native  # noqa: F401
from ._native import (Debug, Dims, MapleError, MapleGraph, MapleLibraryMissing,  # noqa: F401
                      make_debug, make_dims)
