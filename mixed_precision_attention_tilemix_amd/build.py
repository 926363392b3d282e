"""Builds libtilemix.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtilemix.so")
SOURCES = ["api.cpp", "quantize.hip", "pack.hip", "vt_pack.hip", "prefill_fwd.hip", "decode.hip", "route.hip"]

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


def build(verbose: bool = False) -> str:
    """Compile every source into libtilemix.so next to this file; returns its path."""
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError("hipcc failed to build libtilemix.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
