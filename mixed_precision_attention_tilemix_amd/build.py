"""Builds libtilemix.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc, and
libtilemix_peak.so, the matrix-core peak probe that only the benchmark loads."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtilemix.so")
SOURCES = ["api.cpp", "quantize.hip", "pack.hip", "vt_pack.hip", "cache_widen.hip", "prefill_fwd.hip", "decode.hip", "route.hip"]
PEAK_LIB = os.path.join(HERE, "libtilemix_peak.so")
PEAK_SOURCES = ["mfma_peak.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fhip-fp32-correctly-rounded-divide-sqrt",  # the quantizer's scale divisions are exact-rounded
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    root = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(root, "bin", "hipcc")


def _hipcc_shared(out: str, sources, verbose: bool) -> str:
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp] + [os.path.join(CSRC, s) for s in sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError(f"hipcc failed to build {os.path.basename(out)}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile libtilemix.so and libtilemix_peak.so next to this file; returns libtilemix's path."""
    _hipcc_shared(PEAK_LIB, PEAK_SOURCES, verbose)
    return _hipcc_shared(LIB, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
