"""Routed-expert FFN step with an HBM expert cache and PCIe streaming on MI355X.

The compute path is libmoe.so (hand-written HIP kernels for gfx950 behind the C
ABI in include/moe.h); ``_lib`` is its ctypes binding (same function names) and
``runtime`` drives a stack of MoE layers through it.  Build the library with
``python -m routed_expert_streaming_amd.build``.
"""
from . import _lib  # noqa: F401
from ._lib import MoEError  # noqa: F401

__all__ = ["_lib", "MoEError"]
