"""Kimi K2 sparse-MoE feed-forward layer for AMD MI355X (gfx950).

The layer runs in libk2moe.so (hand-written HIP kernels behind the C ABI in
include/k2moe.h); this package holds its build script and a thin ctypes /
PyTorch binding.  Importing the package does not load the library; the first
call into it does, and raises if it has not been built.
"""
from .build import build, lib_path  # noqa: F401


def load():
    from . import _lib
    return _lib.load()
