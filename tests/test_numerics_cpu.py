"""Host-side checks of the numerics sweep: the sweep's workloads have the INT8 coverage they are
named for, and the sweep's exact reference (plain PyTorch fp64) is exact causal attention: it
agrees with the oracle on an all-FP16 route, where the routed score is Q K^T / sqrt(d) exactly."""

import numpy as np
import pytest

import bench
import oracle
from mixed_precision_attention_tilemix_amd import workloads as wl


@pytest.mark.parametrize("cov", [0.0, 0.10, 0.25])
def test_numerics_case_coverage(cov):
    w = wl.numerics_case(2048, cov)
    assert w.q.dtype == np.float16 and w.q.shape == (2048, 24, 128) and w.k.shape == (2048, 8, 128)
    frac = float(w.route.mean())
    if cov == 0.0:
        assert frac == 0.0
    else:
        # 8 KV heads x 32 route rows x 32 groups = 8192 Bernoulli draws
        assert abs(frac - cov) < 4 * np.sqrt(cov * (1 - cov) / w.route.size)


def test_exact_reference_matches_oracle_on_fp16_route():
    oracle.build()
    w = wl.numerics_case(320, 0.0)
    ref = bench.exact_attention_cpu(w)
    out, _, n8, _ = oracle.prepare(w).prefill()
    assert n8 == 0
    assert np.abs(ref - out).max() < 1e-6


def test_exact_reference_causal_first_row():
    # query 0 sees only key 0: O[0] = V[0] of its KV head
    w = wl.numerics_case(64, 0.0)
    ref = bench.exact_attention_cpu(w)
    grp = w.hq // w.hk
    for h in range(w.hq):
        np.testing.assert_array_equal(ref[0, h], w.v[0, h // grp].astype(np.float64))
