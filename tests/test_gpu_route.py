"""GPU parity of the on-device routing policies (tilemix_route_topk_maxabs,
tilemix_route_bernoulli) through the C ABI against the oracle's policies packed by the oracle.

Bar: the route words are integer work, so they must be bit-exact, every word of the output
(sentinel-filled beforehand) included."""

import numpy as np
import pytest
import torch

import oracle
from mixed_precision_attention_tilemix_amd import binding as B
from mixed_precision_attention_tilemix_amd import workloads as wl

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A5A5A5A5A5A5A


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()
    oracle.build()


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def geometry(lq, lk, bm_r, bn_r, g, extra_words=0):
    cu_k, cu_m = _cu(lk), _cu([-(-n // bm_r) for n in lq])
    t_mask = max(1, max(-(-n // (bn_r * g)) for n in lk))
    wpr = -(-t_mask // 64) + extra_words
    return cu_k, cu_m, t_mask, wpr


def fresh_words(hk, rows, wpr):
    w = np.full((hk, rows, wpr), SENTINEL, dtype=np.uint64)
    return _dev(w.view(np.int64))


def got_words(t):
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint64)


def device_topk(cu_k, cu_m, max_k, bn_r, g, pm, wpr, hk, *, k=None, k8=None, k_scale=None):
    words = fresh_words(hk, int(cu_m[-1]), wpr)
    n = B.tilemix_route_workspace_size(batch=len(cu_k) - 1, hkv=hk, max_seqlen_k=max_k,
                                       route_block_n=bn_r, route_group=g)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    B.tilemix_route_topk_maxabs(cu_seqlens_k=_dev(cu_k), cu_mtiles=_dev(cu_m), max_seqlen_k=max_k,
                                route_block_n=bn_r, route_group=g, fp16_per_mille=pm,
                                route_words=words, workspace=ws, k=k, k8=k8, k_scale=k_scale)
    return got_words(words)


TOPK_CASES = {
    # name: (q_lens, k_lens, hk, d, bm_r, bn_r, g, per_mille, extra_words)
    "single_gqa_like": ([3000], [3000], 3, 128, 128, 64, 4, 100, 0),
    "d64_group1": ([700], [700], 2, 64, 64, 64, 1, 250, 0),
    "varlen_empty_and_tails": ([300, 0, 129, 64], [300, 0, 1000, 5000], 2, 128, 64, 64, 2, 300, 1),
    "many_words": ([256], [64 * 130 + 7], 2, 128, 128, 64, 1, 150, 1),
    "budget_zero": ([512], [2048], 2, 128, 128, 128, 1, 0, 0),
    "budget_all": ([512], [2048], 2, 128, 128, 128, 1, 1000, 0),
    "tiny_budget": ([64], [64 * 7], 1, 128, 64, 64, 1, 1, 0),
}


@pytest.mark.parametrize("case", list(TOPK_CASES))
def test_topk_fp16_keys(case):
    lq, lk, hk, d, bm_r, bn_r, g, pm, extra = TOPK_CASES[case]
    cu_k, cu_m, t_mask, wpr = geometry(lq, lk, bm_r, bn_r, g, extra)
    rng = np.random.default_rng(sum(lk) + pm)
    k = rng.standard_normal((int(cu_k[-1]), hk, d)).astype(np.float32)
    k[:, :, rng.choice(d, 3, replace=False)] *= 20.0
    k = k.astype(np.float16)
    got = device_topk(cu_k, cu_m, max(lk), bn_r, g, pm, wpr, hk, k=_dev(k))
    want = oracle.pack_route(oracle.route_topk_maxabs(cu_k, cu_m, hk, d, bn_r, g, pm, k=k, t_mask=t_mask), wpr)
    assert np.array_equal(got, want), case


def test_topk_ties_and_strided_keys():
    # K is the middle third of a packed [T, 3, hk, d] QKV tensor (strided), with many exact ties:
    # values drawn from a few levels so group maxima repeat
    lq, lk, hk, d, bm_r, bn_r, g, pm = [1024], [4096], 4, 128, 128, 64, 1, 200
    cu_k, cu_m, t_mask, wpr = geometry(lq, lk, bm_r, bn_r, g)
    rng = np.random.default_rng(2)
    qkv = rng.choice(np.array([-3, -2, 0.5, 1, 2, 3], dtype=np.float16), size=(4096, 3, hk, d))
    qkv_dev = _dev(qkv)
    k_view = qkv_dev[:, 1]  # strides (3*hk*d, d, 1)
    got = device_topk(cu_k, cu_m, 4096, bn_r, g, pm, wpr, hk, k=k_view)
    want = oracle.pack_route(
        oracle.route_topk_maxabs(cu_k, cu_m, hk, d, bn_r, g, pm, k=qkv[:, 1], t_mask=t_mask), wpr)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("d", [64, 128])
def test_topk_int8_cache(d):
    lq, lk, hk, bm_r, bn_r, g, pm = [2, 1, 3], [5000, 700, 9000], 2, 32, 128, 2, 100
    cu_k, cu_m, t_mask, wpr = geometry(lq, lk, bm_r, bn_r, g)
    rng = np.random.default_rng(d)
    k = (rng.standard_normal((int(cu_k[-1]), hk, d)) * rng.uniform(0.1, 10, (int(cu_k[-1]), hk, 1)))
    k8, ks = oracle.quantize_rows(k.astype(np.float16))  # ks [T, hk]
    got = device_topk(cu_k, cu_m, max(lk), bn_r, g, pm, wpr, hk, k8=_dev(k8), k_scale=_dev(ks.T))
    want = oracle.pack_route(
        oracle.route_topk_maxabs(cu_k, cu_m, hk, d, bn_r, g, pm, k8=k8, k_scale=ks, t_mask=t_mask), wpr)
    assert np.array_equal(got, want)


def test_topk_reproduces_the_32k_gqa_route():
    # the headline workload's route map (top 10 % max|K| groups FP16, built on the host)
    w = wl.make("gqa32k")
    got = device_topk(w.cu_seqlens, w.cu_mtiles, 32768, w.bn_r, w.group, 100, w.words_per_row, w.hk,
                      k=_dev(w.k))
    assert np.array_equal(got, oracle.pack_route(w.route, w.words_per_row))


BERN_CASES = {
    # name: (q_lens, k_lens, hk, bm_r, bn_r, g, per_mille, seed, extra_words)
    "single": ([8192], [8192], 8, 128, 128, 1, 250, 0, 0),
    "varlen_empty": ([100, 0, 3000, 50], [100, 7000, 3000, 0], 4, 64, 64, 2, 200, 12345, 1),
    "many_words": ([128], [64 * 200], 2, 64, 64, 1, 500, 2**63 + 7, 0),
    "budget_zero": ([256], [4096], 2, 128, 64, 1, 0, 1, 0),
    "budget_all": ([256], [4096], 2, 128, 64, 1, 1000, 1, 0),
}


@pytest.mark.parametrize("case", list(BERN_CASES))
def test_bernoulli(case):
    lq, lk, hk, bm_r, bn_r, g, pm, seed, extra = BERN_CASES[case]
    cu_k, cu_m, t_mask, wpr = geometry(lq, lk, bm_r, bn_r, g, extra)
    words = fresh_words(hk, int(cu_m[-1]), wpr)
    B.tilemix_route_bernoulli(cu_seqlens_k=_dev(cu_k), cu_mtiles=_dev(cu_m), max_seqlen_k=max(lk),
                              route_block_n=bn_r, route_group=g, fp16_per_mille=pm, seed=seed,
                              route_words=words)
    got = got_words(words)
    want = oracle.pack_route(oracle.route_bernoulli(cu_k, cu_m, hk, bn_r, g, pm, seed, t_mask=t_mask), wpr)
    assert np.array_equal(got, want), case


@pytest.mark.parametrize("policy", [("topk_maxabs", 400), ("bernoulli", 300, 77)])
@pytest.mark.parametrize("name", ["tiny", "varlen_small", "kv8_small"])
def test_routed_prefill_end_to_end(policy, name):
    # the step with an on-device policy in place of packing; the oracle takes the same policy's map
    from mixed_precision_attention_tilemix_amd.runner import DeviceProblem
    if name == "tiny":
        w = wl.make("tiny")
    elif name == "varlen_small":
        w = wl.custom([300, 1000, 77], 4, 2, 128, bm_r=64, bn_r=64, group=2, seed=6)
    else:
        w = wl.custom([500, 900], 4, 2, 128, bm_r=64, bn_r=64, group=1, kv_int8=True, seed=8)
    if policy[0] == "topk_maxabs" and w.kv_int8:
        k8, ks = oracle.quantize_rows(w.k)
        R = oracle.route_topk_maxabs(w.cu_seqlens, w.cu_mtiles, w.hk, w.d, w.bn_r, w.group, policy[1],
                                     k8=k8, k_scale=ks, t_mask=w.t_mask)
    elif policy[0] == "topk_maxabs":
        R = oracle.route_topk_maxabs(w.cu_seqlens, w.cu_mtiles, w.hk, w.d, w.bn_r, w.group, policy[1],
                                     k=w.k, t_mask=w.t_mask)
    else:
        R = oracle.route_bernoulli(w.cu_seqlens, w.cu_mtiles, w.hk, w.bn_r, w.group, policy[1],
                                   policy[2], t_mask=w.t_mask)
    prob = DeviceProblem(w, out_dtype=torch.float32, route_policy=policy)
    prob.step()
    got = got_words(prob.words)
    assert np.array_equal(got, oracle.pack_route(R, w.words_per_row))
    w.route = R
    ref, _, _, _ = oracle.prepare(w).prefill()
    assert np.abs(prob.out.cpu().numpy() - ref).max() <= 2e-3
