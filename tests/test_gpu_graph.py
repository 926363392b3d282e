"""HIP-graph replay of the decode step (the launch-bound serving loop): a captured step replayed
several times, with the program's own eager work and synchronizations between the replays and new
query tokens written into the input in place, must give bitwise the outputs of the eager step on
the same inputs every time."""

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
