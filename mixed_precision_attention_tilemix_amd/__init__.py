"""Tile-group precision-routed fused prefill attention (TileMix) for AMD Instinct MI355X.

The compute lives in libtilemix.so (HIP kernels for gfx950 behind the C ABI of
include/tilemix.h); ``binding`` is its thin ctypes front end, ``runner`` the torch plumbing
that keeps a workload in device memory, and ``workloads`` the seeded synthetic inputs.
"""

from . import workloads  # noqa: F401

__all__ = ["workloads", "binding", "runner", "build"]
