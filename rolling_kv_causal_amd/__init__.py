"""Sink + rolling-KV chunk attention for AMD MI355X (gfx950): C-ABI library + thin binding.

The library (libsdv2.so, built by ``python -m rolling_kv_causal_amd.build``) holds every step of
the path as hand-written HIP kernels; ``rolling_kv_causal_amd.sdv2`` is its ctypes binding.
"""
from . import sdv2  # noqa: F401
