"""HIP-graph replay of the decode step (the launch-bound serving loop) and of the fused prefill: a
captured step replayed several times, with the program's own eager work and synchronizations
between the replays and new query tokens written into the input in place, must give bitwise the
outputs of the eager step on the same inputs every time."""

import numpy as np
import pytest
import torch

from mixed_precision_attention_tilemix_amd import binding as B
from mixed_precision_attention_tilemix_amd import runner
from mixed_precision_attention_tilemix_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


@pytest.mark.parametrize("fused_q", [True, False])
def test_decode_graph_replays_match_eager(fused_q):
    w = wl.decode_custom([1, 2, 1], [3000, 700, 129], 8, 2, 128, bn_r=64, group=2, seed=5)
    dev = runner.DeviceDecode(w, out_dtype=torch.float32, fused_q=fused_q)
    graph = dev.capture()
    other = runner.DeviceProblem(wl.make("tiny"))  # unrelated eager work between replays
    rng = np.random.default_rng(6)
    for rep in range(4):
        newq = torch.from_numpy(rng.standard_normal(tuple(dev.q.shape)).astype(np.float16)).cuda()
        dev.q.copy_(newq)
        torch.cuda.synchronize()
        graph.replay()
        other.step()
        torch.cuda.synchronize()
        got_o, got_l = dev.out.clone(), dev.lse.clone()
        dev.step()  # eager on the same inputs
        torch.cuda.synchronize()
        assert torch.equal(got_o.view(torch.int32), dev.out.view(torch.int32)), rep
        assert torch.equal(got_l.view(torch.int32), dev.lse.view(torch.int32)), rep
        other.step()


@pytest.mark.parametrize("v_path", [1, 2])
def test_prefill_graph_replays_match_eager(v_path):
    # the fused prefill captured with its pre-pass: on the V^T path (1) the pre-pass zeroes the
    # work-queue counters of the persistent launch, so every replay must find them at zero again
    w = wl.custom([700, 1500, 65], hq=8, hk=2, d=128, bm_r=128, bn_r=128, group=2, p_fp16=0.3, seed=9)
    prob = runner.DeviceProblem(w, out_dtype=torch.float32, fused_q=True)
    prob.quantize()
    prob.route_words()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        prob.attention(v_path=v_path)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        prob.attention(v_path=v_path)
    other = runner.DeviceProblem(wl.make("tiny"))  # unrelated eager work between replays
    rng = np.random.default_rng(10)
    for rep in range(4):
        newq = torch.from_numpy(rng.standard_normal(tuple(prob.q.shape)).astype(np.float16)).cuda()
        prob.q.copy_(newq)
        torch.cuda.synchronize()
        graph.replay()
        other.step()
        torch.cuda.synchronize()
        got_o, got_l = prob.out.clone(), prob.lse.clone()
        prob.attention(v_path=v_path)  # eager on the same inputs
        torch.cuda.synchronize()
        assert torch.equal(got_o.view(torch.int32), prob.out.view(torch.int32)), rep
        assert torch.equal(got_l.view(torch.int32), prob.lse.view(torch.int32)), rep
        other.step()
