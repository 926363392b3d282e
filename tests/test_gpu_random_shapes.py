"""Seeded random shapes through the whole prefill step against the oracle, in full.

Each case draws a batch of sequence lengths (including empty and one-token sequences), a GQA
ratio, head_dim 64 or 128, a route tile (any multiple of 32 rows and 64 keys, so workgroups
straddle route rows at varying offsets), a routing group, causal or not, an fp16 K/V or an INT8
cache, quantize-once or in-kernel Q quantization and fp16 or fp32 output. Both V paths run: their
outputs must be equal bit for bit, and within the parity bars of tests/test_gpu_parity.py of the
oracle (2e-3 max-abs, plus half an fp16 ulp for fp16 output; LSE within 1e-3).
"""

import numpy as np
import pytest
import torch

import oracle
from mixed_precision_attention_tilemix_amd import binding as B
from mixed_precision_attention_tilemix_amd import workloads as wl
from mixed_precision_attention_tilemix_amd.runner import DeviceProblem

pytestmark = pytest.mark.gpu

TOL = 2e-3
LSE_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()
    oracle.build()


def draw(seed):
    """One random configuration (deterministic in the seed)."""
    rng = np.random.default_rng(1000 + seed)
    batch = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.choice([0, 1, 7, 63, 64, 65, 200, 257, 511, 700, 1025], size=batch)]
    if sum(lens) == 0:
        lens[0] = 129
    hk = int(rng.choice([1, 2, 4]))
    hq = hk * int(rng.choice([1, 2, 4]))
    return dict(seqlens=lens, hq=hq, hk=hk, d=int(rng.choice([64, 128])),
                bm_r=32 * int(rng.integers(1, 10)), bn_r=64 * int(rng.integers(1, 4)),
                group=int(rng.integers(1, 4)), causal=bool(rng.integers(0, 2)),
                p_fp16=float(rng.choice([0.0, 0.3, 1.0])), kv_int8=bool(rng.integers(0, 2)),
                seed=seed), bool(rng.integers(0, 2)), bool(rng.integers(0, 2))


CASES = [draw(s) for s in range(80)]


def outputs(prob, v_path):
    prob.out.fill_(float("nan"))
    prob.lse.fill_(float("nan"))
    prob.attention(v_path=v_path)
    torch.cuda.synchronize()
    return prob.out.clone(), prob.lse.clone()


@pytest.mark.parametrize("case", range(len(CASES)))
def test_random_shape_against_oracle(case):
    shape, fused, fp32_out = CASES[case]
    w = wl.custom(**shape)
    prob = DeviceProblem(w, out_dtype=torch.float32 if fp32_out else torch.float16, fused_q=fused)
    prob.quantize()
    prob.route_words()
    o1, l1 = outputs(prob, 1)
    o2, l2 = outputs(prob, 2)
    assert torch.equal(o1.view(torch.int32) if fp32_out else o1.view(torch.int16),
                       o2.view(torch.int32) if fp32_out else o2.view(torch.int16)), f"{shape}: V paths differ"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), f"{shape}: V paths differ (LSE)"
    ref, ref_lse, _, _ = oracle.prepare(w).prefill()
    out = o1.float().cpu().numpy().astype(np.float64)
    tol = TOL + (0.0 if fp32_out else 0.5 * np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64))
    err = np.abs(out - ref)
    assert not (err > tol).any(), f"{shape} fused_q={fused}: max err {err.max():.3e}"
    lse = l1.cpu().numpy()
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin), f"{shape}: LSE finiteness"
    if fin.any():
        assert np.abs(lse[fin] - ref_lse[fin]).max() <= LSE_TOL, f"{shape}: LSE"
