"""Gemma-4 E-series decoder-layer forward for AMD MI355X (gfx950).

The compute path is libg4.so (hand-written HIP kernels behind a C ABI, include/g4.h); `binding` is its
ctypes binding and `model` a small driver that owns descriptors, caches and the workspace.
"""
from . import binding  # noqa: F401

__all__ = ["binding"]
