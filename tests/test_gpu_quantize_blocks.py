"""GPU parity of tilemix_quantize_blocks (block-wise quantization with per-block scales) through
the C ABI against the oracle's block quantizer: codes and scales bit-exact (integer decisions
taken in fp32 on both sides), and the routed prefill on block-quantized Q and K against the
oracle's attention on the same codes (2e-3)."""

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


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


CASES = {
    # name: (lens, heads, d, block_rows)
    "per_token": ([300, 77], 4, 128, 1),
    "route_rows_128": ([1000, 0, 129, 1], 8, 128, 128),
    "route_rows_64_d64": ([700, 64, 65], 4, 64, 64),
    "odd_block": ([999, 5], 2, 128, 100),
    "whole_sequence": ([3000, 200], 2, 128, 100000),
    "long_block": ([5000], 1, 64, 4096),
}


@pytest.mark.parametrize("case", list(CASES))
def test_quantize_blocks_bit_exact(case):
    lens, H, d, blk = CASES[case]
    rng = np.random.default_rng(len(lens) * 1000 + blk)
    T = sum(lens)
    x = (rng.standard_normal((T, H, d)) * rng.uniform(0.01, 40, (T, H, 1))).astype(np.float16)
    if T > 10:
        x[3:9] = 0  # zero rows (and a zero block at block_rows = 1)
    cu = _cu(lens)
    xd = torch.from_numpy(x).cuda()
    x8 = torch.full((T, H, d), 99, dtype=torch.int8, device="cuda")
    sc = torch.full((H, T), -1.0, dtype=torch.float32, device="cuda")
    B.tilemix_quantize_blocks(xd, x8, sc, torch.from_numpy(cu).cuda(), max(lens), blk)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_blocks(x, cu, blk)
    assert np.array_equal(x8.cpu().numpy(), q_ref), case
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), np.ascontiguousarray(s_ref.T).view(np.uint32)), case


def test_quantize_blocks_strided_input():
    # K as the middle third of a packed [T, 3, H, d] tensor
    rng = np.random.default_rng(3)
    lens, H, d, blk = [513, 300], 2, 128, 64
    T = sum(lens)
    qkv = rng.standard_normal((T, 3, H, d)).astype(np.float16)
    dev = torch.from_numpy(qkv).cuda()
    x8 = torch.empty((T, H, d), dtype=torch.int8, device="cuda")
    sc = torch.empty((H, T), dtype=torch.float32, device="cuda")
    cu = _cu(lens)
    B.tilemix_quantize_blocks(dev[:, 1], x8, sc, torch.from_numpy(cu).cuda(), max(lens), blk)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_blocks(qkv[:, 1], cu, blk)
    assert np.array_equal(x8.cpu().numpy(), q_ref)
    assert np.array_equal(sc.cpu().numpy(), s_ref.T)


def oracle_blocks(w, bq, bk):
    q8, qs = oracle.quantize_blocks(w.q, w.cu_seqlens, bq)
    k8, ks = oracle.quantize_blocks(w.k, w.cu_seqlens, bk)
    kw = {}
    if w.kv_int8:
        v8, vs = oracle.quantize_rows(w.v)
        kw = dict(v8=v8, v_scale=vs)
    return oracle.Prepared(q=w.q, k=None if w.kv_int8 else w.k, v=None if w.kv_int8 else w.v,
                           cu_q=w.cu_seqlens, cu_k=w.cu_seqlens, cu_mtiles=w.cu_mtiles, hq=w.hq,
                           hk=w.hk, d=w.d, words=oracle.pack_route(w.route, w.words_per_row),
                           bm_r=w.bm_r, bn_r=w.bn_r, group=w.group, causal=w.causal, q8=q8,
                           q_scale=qs, k8=k8, k_scale=ks, kv_int8=w.kv_int8, **kw)


@pytest.mark.parametrize("name", ["varlen", "kv_int8"])
def test_prefill_on_block_scales(name):
    if name == "varlen":
        w = wl.custom([700, 129, 1000], 8, 2, 128, bm_r=64, bn_r=128, group=1, seed=21)
    else:
        w = wl.custom([900, 300], 4, 2, 128, bm_r=128, bn_r=64, group=2, kv_int8=True, seed=22)
    prob = runner.DeviceProblem(w, out_dtype=torch.float32, scale_blocks=(w.bm_r, w.bn_r))
    prob.step()
    torch.cuda.synchronize()
    prep = oracle_blocks(w, w.bm_r, w.bn_r)
    # the device's block codes are the oracle's
    assert np.array_equal(prob.q8.cpu().numpy(), prep.arrays["q8"])
    assert np.array_equal(prob.k8.cpu().numpy(), prep.arrays["k8"])
    ref, ref_lse, n8, nall = prep.prefill()
    assert n8 > 0
    err = np.abs(prob.out.cpu().numpy() - ref).max()
    assert err <= 2e-3, err


BLOCK_TILE_CASES = {
    # name: (workload factory, (bq, bk))
    "varlen_bk128": (lambda: wl.custom([700, 129, 1000, 64], 8, 2, 128, bm_r=64, bn_r=128, group=1, seed=31),
                     (1, 128)),
    "bk64_d64": (lambda: wl.custom([513, 300], 4, 4, 64, bm_r=64, bn_r=128, group=2, seed=32), (64, 64)),
    "kv_int8_bk256": (lambda: wl.custom([900, 300], 4, 2, 128, bm_r=128, bn_r=64, group=2, kv_int8=True,
                                        seed=33), (128, 256)),
    "zero_k_block": (lambda: _zero_k_block(), (1, 128)),
}


def _zero_k_block():
    w = wl.custom([600], 4, 2, 128, bm_r=128, bn_r=128, route="int8", seed=34)
    w.k[128:256] = 0  # one whole K block of zeros: its scale is 0, next to masked diagonal scores
    return w


@pytest.mark.parametrize("case", list(BLOCK_TILE_CASES))
def test_prefill_block_scale_per_tile(case):
    """With K scales constant over 64-key multiples the kernel takes one K scale per key tile
    (k_scale_block); its outputs meet the 2e-3 bar against the oracle on the same block codes and
    stay within rounding of the per-key path on the same inputs."""
    make, (bq, bk) = BLOCK_TILE_CASES[case]
    w = make()
    tiles = runner.DeviceProblem(w, out_dtype=torch.float32, scale_blocks=(bq, bk))
    assert tiles.k_scale_block == bk
    per_key = runner.DeviceProblem(w, out_dtype=torch.float32, scale_blocks=(bq, bk), k_block_tiles=False)
    assert per_key.k_scale_block == 0
    for prob in (tiles, per_key):
        prob.step()
    torch.cuda.synchronize()
    out_t, out_k = tiles.out.cpu().numpy(), per_key.out.cpu().numpy()
    assert np.isfinite(out_t).all() and np.isfinite(tiles.lse.cpu().numpy()[np.isfinite(per_key.lse.cpu().numpy())]).all()
    ref, _, n8, _ = oracle_blocks(w, bq, bk).prefill()
    assert n8 > 0
    assert np.abs(out_t - ref).max() <= 2e-3, case
    assert np.abs(out_k - ref).max() <= 2e-3, case
    # the two paths associate the three factors (integer score, K scale, per-row factor) in a
    # different order; a last-bit difference in the exponent can flip the fp16 rounding of P,
    # which moves an output by up to half an fp16 ulp of that P times |v|
    assert np.abs(out_t - out_k).max() <= 5e-4, case
