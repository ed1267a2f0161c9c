"""Persistent micro-op dispatch for MI355X (gfx950).

The product is libgpuos.so (C ABI in include/gpuos.h); `gpuos` is its thin
ctypes binding.
"""
from . import gpuos  # noqa: F401

__all__ = ["gpuos"]
