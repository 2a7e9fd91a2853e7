"""Seeded synthetic workloads (shapes and random inputs) for the Gemma-4 E-series layer forward.

Shared by the HIP path's tests and benchmark and by the oracle's tests; holds no step of the method.
"""
from . import configs, gen  # noqa: F401
