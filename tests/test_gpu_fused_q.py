"""GPU checks of fused Q quantization (q8 / q_scale passed as NULL: the prefill and decode kernels
quantize the query rows they load, instead of reading the quantize-once pass's codes).

The fused quantizer uses the same fp32 operations as tilemix_quantize_qk, whose codes are
bit-exact against the oracle, so the bar is bitwise: the int32 accumulators of INT8-routed tiles
equal the oracle's (debug dump), and the outputs and LSE equal those of the quantize-once path
bit for bit; outputs also meet the usual 2e-3 bar against the oracle."""

import numpy as np
import pytest
import torch

import oracle
from mixed_precision_attention_tilemix_amd import binding as B
from mixed_precision_attention_tilemix_amd import runner
from mixed_precision_attention_tilemix_amd import workloads as wl

pytestmark = pytest.mark.gpu



@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()
    oracle.build()


def run(w, fused, **kw):
    prob = runner.DeviceProblem(w, out_dtype=torch.float32, fused_q=fused, **kw)
    prob.step()
    torch.cuda.synchronize()
    return prob


CASES = {
    "tiny": lambda: wl.make("tiny"),
    "varlen_gqa": lambda: wl.custom([300, 1000, 77, 0, 64], 8, 2, 128, bm_r=64, bn_r=64, group=2, seed=3),
    "d64_scaled": lambda: wl.custom([513, 200], 4, 4, 64, bm_r=32, bn_r=64, seed=4, q_std=30.0),
    "kv_int8": lambda: wl.custom([700, 333], 8, 4, 128, bm_r=128, bn_r=128, kv_int8=True, seed=5),
    "zero_rows": lambda: _zero_rows(),
}


def _zero_rows():
    w = wl.custom([200], 2, 1, 128, bm_r=64, bn_r=64, route="int8", seed=6)
    w.q[::7] = 0  # all-zero query rows: scale 0, codes 0
    return w


@pytest.mark.parametrize("case", list(CASES))
def test_prefill_fused_q_equals_quantize_once(case):
    w = CASES[case]()
    once = run(w, False)
    fused = run(w, True)
    assert np.array_equal(once.out.cpu().numpy().view(np.uint32), fused.out.cpu().numpy().view(np.uint32)), case
    assert np.array_equal(once.lse.cpu().numpy().view(np.uint32), fused.lse.cpu().numpy().view(np.uint32)), case
    ref, _, _, _ = oracle.prepare(w).prefill()
    assert np.abs(fused.out.cpu().numpy() - ref).max() <= 2e-3


def test_prefill_fused_q_int32_tiles_bit_exact():
    from test_gpu_parity import compare_dump
    w = wl.custom([640, 200], 4, 2, 128, bm_r=64, bn_r=64, group=1, seed=8)
    prob = run(w, True)
    for head in (0, w.hq - 1):
        assert compare_dump(w, prob, head, 0, w.total_mtiles) > 0


@pytest.mark.parametrize("d", [64, 128])
def test_decode_fused_q_equals_quantize_once(d):
    w = wl.decode_custom([1, 3, 2, 0], [3000, 700, 64, 10], 8, 2, d, bn_r=64, group=2, seed=12)
    outs = []
    for fused in (False, True):
        dev = runner.DeviceDecode(w, out_dtype=torch.float32, fused_q=fused)
        dev.step()
        torch.cuda.synchronize()
        outs.append((dev.out.cpu().numpy(), dev.lse.cpu().numpy()))
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32))
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
