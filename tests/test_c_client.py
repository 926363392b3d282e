"""The C ABI from a plain C program (tests/c/prefill_client.c, built with gcc against
include/tilemix.h, libtilemix.so and the HIP runtime C API): argument validation on the CPU, and
one routed prefill on the GPU compared with the oracle (2e-3). The client runs as a child
process and allocates its own device memory."""

import os
import subprocess

import numpy as np
import pytest

import oracle
from mixed_precision_attention_tilemix_amd import binding as B
from mixed_precision_attention_tilemix_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mixed_precision_attention_tilemix_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_client(tmp_path):
    if not os.path.exists(B.LIB_PATH):
        from mixed_precision_attention_tilemix_amd import build
        build.build()
    exe = str(tmp_path / "prefill_client")
    subprocess.check_call(["gcc", "-std=c99", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
                           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                           os.path.join(ROOT, "tests", "c", "prefill_client.c"), "-L", PKG,
                           "-L", os.path.join(ROCM, "lib"), "-ltilemix", "-lamdhip64",
                           f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe])
    return exe


def test_c_client_validation(tmp_path):
    exe = build_client(tmp_path)
    r = subprocess.run([exe, "--validate"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failure(s)" in r.stdout


@pytest.mark.gpu
def test_c_client_prefill_matches_oracle(tmp_path):
    exe = build_client(tmp_path)
    w = wl.custom([300, 77, 513], 8, 2, 128, bm_r=64, bn_r=64, group=2, seed=41)
    d = tmp_path / "case"
    d.mkdir()
    total_m = w.total_mtiles
    meta = [w.batch, w.hq, w.hk, w.d, w.total, w.total, w.bm_r, w.bn_r, w.group, int(w.causal),
            w.t_mask, w.words_per_row, total_m, max(w.seqlens), max(w.seqlens)]
    (d / "meta.txt").write_text(" ".join(str(x) for x in meta) + "\n")
    for name, arr in (("q", w.q), ("k", w.k), ("v", w.v), ("route", w.route), ("cu_q", w.cu_seqlens),
                      ("cu_k", w.cu_seqlens), ("cu_m", w.cu_mtiles)):
        np.ascontiguousarray(arr).tofile(str(d / f"{name}.bin"))
    r = subprocess.run([exe, str(d)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    out = np.fromfile(str(d / "out.bin"), dtype=np.float32).reshape(w.total, w.hq, w.d)
    oracle.build()
    ref = oracle.prepare(w).prefill()[0]
    err = float(np.abs(out.astype(np.float64) - ref).max())
    print(r.stdout.strip(), f"max err {err:.2e}")
    assert err <= 2e-3, err
