"""GPU edge cases of tilemix_prefill_fwd through the C ABI against the oracle: varlen batches
whose query and key lengths differ per sequence (bottom-right causal alignment, queries with no
legal key get O = 0 and LSE = -inf), non-causal L_q != L_k, a 64:1 GQA group, and the same
shapes over an INT8 K/V cache. Bars as in test_gpu_parity (2e-3 on outputs, 1e-3 on LSE)."""

import numpy as np
import pytest
import torch

import oracle
from mixed_precision_attention_tilemix_amd import binding as B

pytestmark = pytest.mark.gpu

TOL, LSE_TOL = 2e-3, 1e-3


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()
    oracle.build()


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def run_case(lq, lk, hq, hk, d, bm, bn, g, causal, kv_int8, seed, v_path=0, ws_fill=None):
    rng = np.random.default_rng(seed)
    Tq, Tk = sum(lq), sum(lk)
    q = rng.standard_normal((Tq, hq, d)).astype(np.float16)
    k = (rng.standard_normal((Tk, hk, d)) * 2).astype(np.float16)
    v = rng.standard_normal((Tk, hk, d)).astype(np.float16)
    cu_q, cu_k = _cu(lq), _cu(lk)
    cu_m = _cu([-(-n // bm) for n in lq])
    t_mask = max(1, max(-(-n // (bn * g)) for n in lk))
    wpr = -(-t_mask // 64)
    R = (rng.random((hk, int(cu_m[-1]), t_mask)) < 0.6).astype(np.uint8)
    q8, qs = oracle.quantize_rows(q)
    k8, ks = oracle.quantize_rows(k)
    kw = {}
    if kv_int8:
        v8, vs = oracle.quantize_rows(v)
        kw = dict(v8=v8, v_scale=vs)
    prep = oracle.Prepared(q=q, k=None if kv_int8 else k, v=None if kv_int8 else v, cu_q=cu_q, cu_k=cu_k,
                           cu_mtiles=cu_m, hq=hq, hk=hk, d=d, words=oracle.pack_route(R, wpr), bm_r=bm,
                           bn_r=bn, group=g, causal=causal, q8=q8, q_scale=qs, k8=k8, k_scale=ks,
                           kv_int8=kv_int8, **kw)
    ref, ref_lse, _, _ = prep.prefill()

    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    dk8, dks = t(k8), t(ks.T)
    dv8 = dvs = None
    if kv_int8:
        dv8, dvs = t(kw["v8"]), t(kw["v_scale"].T)
    words = torch.empty((hk, int(cu_m[-1]), wpr), dtype=torch.int64, device="cuda")
    B.tilemix_pack_route_mask(t(R).view(-1, t_mask), words.view(-1, wpr))
    out = torch.empty((Tq, hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((hq, Tq), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(256, B.tilemix_prefill_workspace_size(batch=len(lq), hkv=hk, head_dim=d, total_k=Tk,
                                                               kv_int8=kv_int8)), dtype=torch.uint8, device="cuda")
    if ws_fill is not None:
        ws.fill_(ws_fill)
    B.tilemix_prefill_fwd(q=t(q), q8=None, q_scale=None, k8=dk8, k_scale=dks, k=None if kv_int8 else t(k),
                          v=None if kv_int8 else t(v), v8=dv8, v_scale=dvs, route_words=words,
                          cu_seqlens_q=t(cu_q), cu_seqlens_k=t(cu_k), cu_mtiles=t(cu_m),
                          max_seqlen_q=max(lq), max_seqlen_k=max(lk), route_block_m=bm, route_block_n=bn,
                          route_group=g, causal=causal, out=out, lse=lse, workspace=ws, v_path=v_path)
    torch.cuda.synchronize()
    got, got_lse = out.cpu().numpy(), lse.cpu().numpy()
    err = np.abs(got.astype(np.float64) - ref).max()
    assert err <= TOL, err
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(got_lse), fin)
    if fin.any():
        assert np.abs(got_lse[fin] - ref_lse[fin]).max() <= LSE_TOL
    return got, got_lse, cu_q, cu_k


@pytest.mark.parametrize("kv_int8", [False, True])
def test_varlen_more_queries_than_keys(kv_int8):
    # sequence 0: 200 queries, 70 keys (the first 130 queries see no key); sequence 1: 64 / 1000;
    # sequence 2: 5 / 5; sequence 3: 33 queries, 0 keys
    lq, lk = [200, 64, 5, 33], [70, 1000, 5, 0]
    got, got_lse, cu_q, _ = run_case(lq, lk, 4, 2, 128, 64, 64, 1, True, kv_int8, seed=31)
    s0 = slice(cu_q[0], cu_q[0] + 130)
    assert np.all(got[s0] == 0) and np.all(np.isneginf(got_lse[:, s0]))
    s3 = slice(cu_q[3], cu_q[4])
    assert np.all(got[s3] == 0) and np.all(np.isneginf(got_lse[:, s3]))


@pytest.mark.parametrize("kv_int8", [False, True])
def test_non_causal_unequal_lengths(kv_int8):
    run_case([100, 300], [777, 64], 4, 4, 64, 32, 128, 2, False, kv_int8, seed=32)


def test_gqa_64_to_1():
    run_case([300], [300], 64, 1, 128, 64, 64, 1, True, False, seed=33)


def draw_unequal(seed):
    """Random varlen batch whose query and key lengths differ per sequence (deterministic)."""
    rng = np.random.default_rng(5000 + seed)
    n = int(rng.integers(1, 5))
    lens = [0, 1, 31, 64, 65, 255, 256, 300, 513, 1000]
    lq = [int(x) for x in rng.choice(lens, size=n)]
    lk = [int(x) for x in rng.choice(lens, size=n)]
    if sum(lq) == 0:
        lq[0] = 97
    if sum(lk) == 0:
        lk[-1] = 97
    hk = int(rng.choice([1, 2, 4]))
    return dict(lq=lq, lk=lk, hq=hk * int(rng.choice([1, 2, 4])), hk=hk, d=int(rng.choice([64, 128])),
                bm=32 * int(rng.integers(1, 9)), bn=64 * int(rng.integers(1, 4)), g=int(rng.integers(1, 4)),
                causal=bool(rng.integers(0, 2)), kv_int8=bool(rng.integers(0, 2)), seed=6000 + seed)


@pytest.mark.parametrize("seed", range(40))
def test_random_unequal_lengths(seed):
    # bottom-right causal alignment with L_q > L_k (rows without a legal key) and L_q < L_k, in
    # both V paths, which must agree bit for bit
    c = draw_unequal(seed)
    o1, l1, _, _ = run_case(**c, v_path=1)
    o2, l2, _, _ = run_case(**c, v_path=2)
    assert np.array_equal(o1.view(np.int32), o2.view(np.int32)), c
    assert np.array_equal(l1.view(np.int32), l2.view(np.int32)), c


def test_vt_path_workspace_garbage():
    # the V^T path keeps its work-queue counters in the workspace; whatever the workspace holds on
    # entry, the pre-pass zeroes them, so a workspace filled with 0x7f bytes gives the same outputs
    lq = lk = [900, 300]
    first = run_case(lq, lk, 8, 2, 128, 128, 128, 1, True, False, seed=40, v_path=1)
    again = run_case(lq, lk, 8, 2, 128, 128, 128, 1, True, False, seed=40, v_path=1, ws_fill=0x7F)
    assert np.array_equal(first[0].view(np.int32), again[0].view(np.int32))
    assert np.array_equal(first[1].view(np.int32), again[1].view(np.int32))
