"""Host-side checks of the numerics sweep: the sweep's workloads have the INT8 coverage they are
named for, and the sweep's exact reference (plain PyTorch fp64) is exact causal attention: it
agrees with the oracle on an all-FP16 route, where the routed score is Q K^T / sqrt(d) exactly.
Also the pages' FP16-state variant, emulated on the CPU (the kernels keep an fp32 state)."""

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


def online_attention(S, V, bn, state):
    """The online-softmax recurrence (TileMix paper, Section 3.1) over key blocks of width bn,
    with P rounded to fp16 for P.V (Section 4.3) and the shared state (m, z, O) stored in `state`
    after every block: np.float16 is the pages' FP16 state (Section 4.3), np.float64 the exact
    reference. Masked scores are -inf; returns O / z."""
    L = S.shape[0]
    m = np.full(L, -np.inf)
    z = np.zeros(L)
    O = np.zeros((L, V.shape[1]))
    for j0 in range(0, S.shape[1], bn):
        Sb = S[:, j0:j0 + bn]
        m_new = np.maximum(m, Sb.max(axis=1)).astype(state).astype(np.float64)
        alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
        P = np.where(np.isfinite(Sb), np.exp(Sb - m_new[:, None]), 0.0).astype(np.float16).astype(np.float64)
        z = (alpha * z + P.sum(axis=1)).astype(state).astype(np.float64)
        O = (alpha[:, None] * O + P @ V[j0:j0 + bn]).astype(state).astype(np.float64)
        m = m_new
    return O / z[:, None]


@pytest.mark.parametrize("L", [1024, 4096])
def test_fp16_state_variant_study(L):
    """The pages' FP16-state variant (their Appendix G.3 / G.4 accumulation study), emulated on
    the CPU: keeping (m, z, O) in fp16 moves the output by less than the parity bar and by less
    than routing a quarter of the tile groups to INT8 does."""
    oracle.build()
    d = 128
    w = wl.numerics_case(L, 0.0)
    q = w.q[:, 0].astype(np.float64)
    k = w.k[:, 0].astype(np.float64)
    v = w.v[:, 0].astype(np.float64)
    S = np.where(np.tril(np.ones((L, L), bool)), (q @ k.T) / np.sqrt(d), -np.inf)
    exact = bench.exact_attention_cpu(w)[:, 0]
    o32 = online_attention(S, v, 64, np.float64)
    o16 = online_attention(S, v, 64, np.float16)
    w25 = wl.numerics_case(L, 0.25)
    o_int8 = oracle.prepare(w25).prefill()[0][:, 0]
    dev32 = np.abs(o32 - exact).mean()
    dev16 = np.abs(o16 - exact).mean()
    dev_int8 = np.abs(o_int8 - exact).mean()
    print(f"L={L}: mean |O - O_exact|: fp32 state {dev32:.2e}, fp16 state {dev16:.2e}, "
          f"25% INT8 groups {dev_int8:.2e}")
    assert np.abs(o16 - exact).max() < 2e-3
    assert dev32 < dev16 < dev_int8
