"""GPU checks that tie the other instances of the fused prefill kernel to the production one.

  * The single-buffered instance (debug_sync_stages) loads each key tile into the one LDS stage
    and waits for it before computing on it; the production kernel streams tile n+1 into the
    second stage while tile n is computed. Both must give the same O and LSE bit for bit: a
    staging race in the production kernel would show as a difference (a race detector by diff).
  * The debug-dump instance computes the same O and LSE as the production instance, bit for bit,
    so that the int32 tiles it dumps (checked bit-exact against the oracle elsewhere) are the
    tiles behind the production outputs.
  * The FP16-state instance (state_fp16; the TileMix page, Section 4.3 and Appendix G.3) keeps the
    online-softmax state in binary16 between 64-key tiles. It is held to the same 2e-3 bar
    against the oracle as the production kernel, and must actually differ from it.
  * The two ways of reading V (v_path 1: V^T tiles from a pre-pass; v_path 2: V rows staged as
    they are and transposed by the LDS reads) give the same O and LSE bit for bit, in every
    instance.
"""

import functools

import numpy as np
import pytest
import torch

import oracle
from mixed_precision_attention_tilemix_amd import binding as B
from mixed_precision_attention_tilemix_amd import workloads as wl
from mixed_precision_attention_tilemix_amd.runner import DeviceProblem

pytestmark = pytest.mark.gpu

TOL = 2e-3
SENTINEL = np.iinfo(np.int32).min


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()
    oracle.build()


@functools.lru_cache(maxsize=None)
def named(name):
    return wl.make(name)


def outputs(prob, **kw):
    """O and LSE of one launch of the fused kernel (buffers poisoned first)."""
    prob.out.fill_(float("nan"))
    prob.lse.fill_(float("nan"))
    prob.attention(**kw)
    torch.cuda.synchronize()
    return prob.out.clone(), prob.lse.clone()


def assert_bitwise(a, b, what):
    (oa, la), (ob, lb) = a, b
    assert not torch.isnan(oa).any(), f"{what}: unwritten output"
    same_o = torch.equal(oa.view(torch.int16) if oa.dtype == torch.float16 else oa.view(torch.int32),
                         ob.view(torch.int16) if ob.dtype == torch.float16 else ob.view(torch.int32))
    assert same_o, f"{what}: O differs (max |diff| {(oa.float() - ob.float()).abs().max().item():.3e})"
    assert torch.equal(la.view(torch.int32), lb.view(torch.int32)), f"{what}: LSE differs"


SHAPES = [
    dict(seqlens=[256], hq=2, hk=2, d=64, bm_r=64, bn_r=64, group=1),
    dict(seqlens=[37, 130, 1, 64], hq=4, hk=2, d=64, bm_r=32, bn_r=64, group=2),
    dict(seqlens=[300, 77], hq=6, hk=2, d=128, bm_r=64, bn_r=128, group=1, causal=False),
    dict(seqlens=[0, 150, 0, 9], hq=2, hk=1, d=128, bm_r=32, bn_r=64, group=1),
    dict(seqlens=[513, 200], hq=8, hk=2, d=128, bm_r=128, bn_r=128, group=3),
    dict(seqlens=[700, 333], hq=4, hk=1, d=128, bm_r=64, bn_r=64, group=1, kv_int8=True),
]


def ids(s):
    return "-".join(f"{k}{v}" for k, v in s.items() if k not in ("hq", "hk")).replace(" ", "")


# ----------------------------------------------------------------------------- single-buffered

@pytest.mark.parametrize("shape", SHAPES, ids=[ids(s) for s in SHAPES])
def test_sync_instance_bitwise_small(shape):
    w = wl.custom(seed=41, **shape)
    for fused in (False, True):
        prob = DeviceProblem(w, fused_q=fused)
        prob.quantize()
        prob.route_words()
        prod = outputs(prob, v_path=1)
        for v_path in (1, 2):
            tag = f"{ids(shape)} fused_q={fused} v_path={v_path}"
            if v_path == 2:
                assert_bitwise(prod, outputs(prob, v_path=2), tag + " (production against v_path=1)")
            assert_bitwise(prod, outputs(prob, debug_sync_stages=True, v_path=v_path), tag)


V_PATH_SHAPES = SHAPES + [
    dict(seqlens=[700, 300], hq=4, hk=2, d=128, bm_r=96, bn_r=64, group=2),
    dict(seqlens=[160, 65, 1], hq=2, hk=2, d=64, bm_r=32, bn_r=64, group=1, kv_int8=True, causal=False),
]


@pytest.mark.parametrize("shape", V_PATH_SHAPES, ids=[ids(s) for s in V_PATH_SHAPES])
def test_v_paths_bitwise_all_instances(shape):
    """Both V paths in the production, block-scale, dump and FP16-state instances: equal bit for
    bit (the dump tiles too), and the automatic choice equal to both."""
    w = wl.custom(seed=43, **shape)
    prob = DeviceProblem(w, fused_q=True)
    prob.quantize()
    prob.route_words()
    auto = outputs(prob)
    for kw in ({}, dict(state_fp16=True)):
        a, b = outputs(prob, v_path=1, **kw), outputs(prob, v_path=2, **kw)
        assert_bitwise(a, b, f"{ids(shape)} {kw}")
        if not kw:
            assert_bitwise(auto, a, f"{ids(shape)} automatic choice")
    ntiles = -(-max(w.seqlens) // w.bn_r) if w.seqlens else 1
    dumps = []
    for v_path in (1, 2):
        d = torch.full((w.total_mtiles, max(ntiles, 1), w.bm_r, w.bn_r), SENTINEL, dtype=torch.int32, device="cuda")
        o = outputs(prob, v_path=v_path, debug_s32=d, debug_head=w.hq - 1, debug_mtile_begin=0,
                    debug_mtile_count=w.total_mtiles)
        assert_bitwise(auto, o, f"{ids(shape)} dump instance v_path={v_path}")
        dumps.append(d)
    assert torch.equal(dumps[0], dumps[1]), f"{ids(shape)}: dumped tiles differ between V paths"
    kb = DeviceProblem(w, fused_q=True, scale_blocks=(1, 128))
    kb.quantize()
    kb.route_words()
    assert_bitwise(outputs(kb, v_path=1), outputs(kb, v_path=2), f"{ids(shape)} block-scale instance")


@pytest.mark.parametrize("name", ["mha8k", "gqa32k"])
def test_v_paths_bitwise_full_size(name):
    """Whole outputs of a workload that takes the direct path (mha8k) and one that takes the V^T
    path (gqa32k) by default, forced through the other path, in the configuration bench.py times."""
    w = named(name)
    prob = DeviceProblem(w, out_dtype=torch.float16, fused_q=True)
    prob.quantize()
    prob.route_words()
    assert_bitwise(outputs(prob, v_path=1), outputs(prob, v_path=2), name)
    del prob
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["gqa32k", "varlen64k"])
def test_sync_instance_bitwise_full_size(name):
    """Whole outputs of the full-size workloads, in the configuration bench.py times (Q quantized
    inside the fused kernel, fp16 output) and with the quantize-once pass and fp32 output."""
    w = named(name)
    for fused, dtype in ((True, torch.float16), (False, torch.float32)):
        prob = DeviceProblem(w, out_dtype=dtype, fused_q=fused)
        prob.quantize()
        prob.route_words()
        prod = outputs(prob)
        sync = outputs(prob, debug_sync_stages=True)
        assert_bitwise(prod, sync, f"{name} fused_q={fused}")
        del prob, prod, sync
        torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- dump instance

@pytest.mark.parametrize("name", ["gqa32k", "kvint8_128k"])
def test_dump_instance_matches_production(name):
    """O and LSE of the dump instance equal the production instance's bit for bit, with the dump
    taken for the first, middle and last route rows of the last head."""
    w = named(name)
    ntiles = -(-max(w.seqlens) // w.bn_r)
    last = w.total_mtiles - 1
    for fused in (False, True):
        prob = DeviceProblem(w, out_dtype=torch.float16 if fused else torch.float32, fused_q=fused)
        prob.quantize()
        prob.route_words()
        prod = outputs(prob)
        for m0 in (0, last // 2, last):
            dump = torch.full((1, ntiles, w.bm_r, w.bn_r), SENTINEL, dtype=torch.int32, device="cuda")
            got = outputs(prob, debug_s32=dump, debug_head=w.hq - 1, debug_mtile_begin=m0,
                          debug_mtile_count=1)
            assert_bitwise(prod, got, f"{name} fused_q={fused} route row {m0}")
        del prob, prod
        torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- FP16 state

def check_out(out, ref, what):
    err = np.abs(out.astype(np.float64) - ref)
    assert err.max() <= TOL, f"{what}: max err {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}"
    return float(err.max())


@pytest.mark.parametrize("L", [1024, 4096])
@pytest.mark.parametrize("frac", [0.0, 0.25])
def test_fp16_state_parity_numerics_cases(L, frac):
    """The accumulation-study inputs (INT8 coverage 0 and 25 %, 1k and 4k tokens) with the state
    in binary16: within 2e-3 of the oracle, and not equal to the fp32-state output."""
    w = wl.numerics_case(L, frac)
    ref, _, _, _ = oracle.prepare(w).prefill()
    prob = DeviceProblem(w)
    prob.quantize()
    prob.route_words()
    o32, _ = outputs(prob)
    o16, l16 = outputs(prob, state_fp16=True)
    err16 = check_out(o16.cpu().numpy(), ref, f"fp16 state L={L} frac={frac}")
    err32 = check_out(o32.cpu().numpy(), ref, f"fp32 state L={L} frac={frac}")
    assert torch.isfinite(l16).all()
    assert not torch.equal(o16, o32), "state_fp16 changed nothing"
    print(f"L={L} INT8 {frac:.0%}: max |O - oracle| fp32 state {err32:.2e}, fp16 state {err16:.2e}")


@pytest.mark.parametrize("shape", SHAPES, ids=[ids(s) for s in SHAPES])
def test_fp16_state_parity_small(shape):
    w = wl.custom(seed=42, **shape)
    ref, ref_lse, _, _ = oracle.prepare(w).prefill()
    prob = DeviceProblem(w)
    prob.quantize()
    prob.route_words()
    o16, l16 = outputs(prob, state_fp16=True)
    check_out(o16.cpu().numpy(), ref, ids(shape))
    fin = np.isfinite(ref_lse)
    lse = l16.cpu().numpy()
    assert np.array_equal(np.isfinite(lse), fin)
    if fin.any():  # the row sum is rounded to binary16 (2^-11 relative) after every tile
        assert np.abs(lse[fin] - ref_lse[fin]).max() <= 2e-3
