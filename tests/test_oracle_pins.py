"""Pins of the CPU oracle against facts fixed by the TileMix paper and by mathematics.

Nothing here re-types the oracle's own loops. Each test checks the oracle against something
else: hand-worked golden cases (tests/golden/), textbook attention through numpy matrix
products, closed forms (V = ones, Q = 0, first row), structural identities (GQA = repeated
heads, varlen = independent sequences, grouping = repeated bits) and an independent numpy
implementation of the online-softmax recurrence of Section 3.1 on brute-force tiny inputs.
"""

import itertools
import json
import os

import numpy as np
import pytest

from mixed_precision_attention_tilemix_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
# the oracle computes in fp64 and stores fp32: one fp32 rounding (2^-24 relative) separates it from fp64
F32 = 2.0 ** -24 * 1.01


# ----------------------------------------------------------------------------- helpers (numpy)

def textbook(q, k, v, cu_q, cu_k, hq, hk, causal, scale=None):
    """softmax(Q K^T / sqrt(d)) V per sequence and head, fp64 numpy (Section 3.1 definition)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[-1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.zeros(q.shape, dtype=np.float64)
    lse = np.full((hq, q.shape[0]), -np.inf)
    rep = hq // hk
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        Lq, Lk = q1 - q0, k1 - k0
        if Lq == 0:
            continue
        for h in range(hq):
            S = q[q0:q1, h] @ k[k0:k1, h // rep].T * scale
            if causal:
                ii = np.arange(Lq)[:, None]
                jj = np.arange(Lk)[None, :]
                S = np.where(jj <= ii + (Lk - Lq), S, -np.inf)
            M = S.max(axis=1, keepdims=True) if Lk else np.full((Lq, 1), -np.inf)
            has = np.isfinite(M[:, 0])
            P = np.where(has[:, None], np.exp(S - np.where(has[:, None], M, 0.0)), 0.0)
            l = P.sum(axis=1)
            O = np.where(has[:, None], (P @ v[k0:k1, h // rep]) / np.where(has, l, 1.0)[:, None], 0.0)
            out[q0:q1, h] = O
            lse[h, q0:q1] = np.where(has, M[:, 0] + np.log(np.where(has, l, 1.0)), -np.inf)
    return out, lse


def expand_route(route_hk, seqlens, bm_r, bn_r, group):
    """Element-wise route map per sequence from R[row, g] by repetition (no bit arithmetic)."""
    maps = []
    r0 = 0
    for L in seqlens:
        nt = -(-L // bm_r)
        R = route_hk[r0:r0 + nt]
        r0 += nt
        E = np.repeat(np.repeat(R, bm_r, axis=0), bn_r * group, axis=1)
        need = -(-L // (bn_r * group)) * bn_r * group
        if E.shape[1] < need:
            E = np.pad(E, ((0, 0), (0, need - E.shape[1])))
        maps.append(E[:L, :L].astype(bool))
    return maps


def dequant(x8, s):
    return x8.astype(np.float64) * s.astype(np.float64)[..., None]


def run_oracle(oracle, w, **kw):
    prep = oracle.prepare(w, **kw)
    out, lse, n8, nall = prep.prefill()
    return out, lse, n8, nall, prep


# ----------------------------------------------------------------------------- fp16 decoding

def test_fp16_decode_matches_ieee_binary16(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle_mod.decode_fp16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ----------------------------------------------------------------------------- quantizer

def test_quantize_golden_cases(oracle_mod):
    cases = json.load(open(os.path.join(GOLDEN, "quantize_cases.json")))["cases"]
    for c in cases:
        x = np.array(c["x"], dtype=np.float16)[None]
        q, s = oracle_mod.quantize_rows(x)
        assert q[0].tolist() == c["q"], c["why"]
        if "scale" in c:
            exp = np.float32(c["scale"])
        else:
            a, b = c["scale_over"]
            exp = np.float32(a) / np.float32(b)
        assert s[0] == exp, c["why"]


@pytest.mark.parametrize("d", [64, 128])
def test_quantize_properties(oracle_mod, d):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((500, d)) * rng.uniform(0.01, 30, (500, 1))).astype(np.float16)
    x[3] = 0
    x[4, :] = 0
    x[4, 5] = -3.0
    q, s = oracle_mod.quantize_rows(x)
    xf = x.astype(np.float64)
    amax = np.abs(xf).max(axis=1)
    nz = amax > 0
    # scale is a/127 rounded to fp32
    assert np.array_equal(s[nz], (amax[nz].astype(np.float32) / np.float32(127)))
    assert np.all(s[~nz] == 0) and np.all(q[~nz] == 0)
    # the largest magnitude element maps to +-127 with its sign
    am = np.abs(xf).argmax(axis=1)
    top = q[np.arange(len(q)), am]
    assert np.all(np.abs(top[nz]) == 127)
    assert np.all(np.sign(top[nz]) == np.sign(xf[np.arange(len(q)), am][nz]))
    # nearest grid point: |x - delta*q| <= delta/2 (+ fp32 rounding of the product)
    err = np.abs(xf - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err[nz] <= s[nz, None] * (0.5 + 1e-5))
    assert np.all(np.abs(q) <= 127)


def test_quantize_power_of_two_invariance(oracle_mod):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 128)).astype(np.float16)
    q1, s1 = oracle_mod.quantize_rows(x)
    q2, s2 = oracle_mod.quantize_rows((x.astype(np.float32) * 4).astype(np.float16))
    assert np.array_equal(q1, q2)
    assert np.array_equal(s2, s1 * np.float32(4))


# ----------------------------------------------------------------------------- pack / decode

def test_pack_golden_cases(oracle_mod):
    cases = json.load(open(os.path.join(GOLDEN, "pack_cases.json")))["cases"]
    for c in cases:
        R = np.array(c["R"], dtype=np.uint8)[None]
        words = oracle_mod.pack_route(R)
        assert [int(w) for w in words[0]] == [int(x) for x in c["words"]], c["why"]


def test_pack_roundtrip_and_rejects(oracle_mod):
    rng = np.random.default_rng(0)
    for t in (1, 5, 63, 64, 65, 128, 130):
        R = (rng.random((7, t)) < 0.5).astype(np.uint8)
        W = oracle_mod.pack_route(R)
        assert W.shape == (7, -(-t // 64))
        back = np.array([[(int(W[r, g >> 6]) >> (g & 63)) & 1 for g in range(t)] for r in range(7)])
        assert np.array_equal(back, R)
        # unused high bits stay zero
        for r in range(7):
            full = sum(int(W[r, w]) << (64 * w) for w in range(W.shape[1]))
            assert full >> t == 0
    with pytest.raises(ValueError):
        oracle_mod.pack_route(np.array([[0, 2, 1]], dtype=np.uint8))


# ----------------------------------------------------------------------------- attention closed forms

SHAPES = [
    dict(seqlens=[256], hq=2, hk=2, d=64, bm_r=64, bn_r=64, group=1, causal=True),
    dict(seqlens=[37, 130, 1, 64], hq=4, hk=2, d=64, bm_r=32, bn_r=32, group=2, causal=True),
    dict(seqlens=[200, 77], hq=6, hk=2, d=128, bm_r=64, bn_r=32, group=3, causal=False),
    dict(seqlens=[0, 150, 0, 9], hq=2, hk=1, d=32, bm_r=16, bn_r=16, group=1, causal=True),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_all_fp16_mask_is_textbook_attention(oracle_mod, shape):
    w = wl.custom(route="fp16", seed=1, **shape)
    out, lse, n8, nall, _ = run_oracle(oracle_mod, w)
    ref, ref_lse = textbook(w.q, w.k, w.v, w.cu_seqlens, w.cu_seqlens, w.hq, w.hk, w.causal)
    assert n8 == 0 and nall == w.legal_pairs() * w.hq
    np.testing.assert_allclose(out, ref, rtol=F32, atol=1e-12)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin)
    np.testing.assert_allclose(lse[fin], ref_lse[fin], rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("shape", SHAPES)
def test_all_int8_mask_is_uniform_int8_attention(oracle_mod, shape):
    """delta_q delta_k sum(q8 k8) = sum((delta_q q8)(delta_k k8)): uniform INT8 attention is
    textbook attention on the dequantized Q and K (Section 3.2 product identity)."""
    w = wl.custom(route="int8", seed=2, **shape)
    out, lse, n8, nall, _ = run_oracle(oracle_mod, w)
    q8, qs = oracle_mod.quantize_rows(w.q)
    k8, ks = oracle_mod.quantize_rows(w.k)
    ref, _ = textbook(dequant(q8, qs), dequant(k8, ks), w.v, w.cu_seqlens, w.cu_seqlens,
                      w.hq, w.hk, w.causal)
    assert n8 == nall == w.legal_pairs() * w.hq
    np.testing.assert_allclose(out, ref, rtol=F32, atol=1e-12)


def test_int8_differs_from_fp16(oracle_mod):
    """Guards against a path that ignores the route bits: the two paths must disagree."""
    s = SHAPES[0]
    a = run_oracle(oracle_mod, wl.custom(route="fp16", seed=3, **s))[0]
    b = run_oracle(oracle_mod, wl.custom(route="int8", seed=3, **s))[0]
    assert np.abs(a - b).max() > 1e-4


@pytest.mark.parametrize("route", ["fp16", "int8", None])
def test_v_ones_gives_ones(oracle_mod, route):
    w = wl.custom(route=route, seed=4, **SHAPES[1])
    w.v[:] = np.float16(1.0)
    out = run_oracle(oracle_mod, w)[0]
    np.testing.assert_allclose(out, 1.0, rtol=F32, atol=1e-13)


@pytest.mark.parametrize("route", ["fp16", "int8", None])
def test_zero_query_gives_causal_prefix_mean(oracle_mod, route):
    w = wl.custom(route=route, seed=5, **SHAPES[1])
    w.q[:] = 0
    out = run_oracle(oracle_mod, w)[0]
    cu = w.cu_seqlens
    v = w.v.astype(np.float64)
    for b in range(w.batch):
        L = w.seqlens[b]
        if L == 0:
            continue
        vb = v[cu[b]:cu[b + 1]]
        mean = np.cumsum(vb, axis=0) / np.arange(1, L + 1)[:, None, None]
        for h in range(w.hq):
            np.testing.assert_allclose(out[cu[b]:cu[b + 1], h], mean[:, h // (w.hq // w.hk)],
                                       rtol=F32, atol=1e-12)


@pytest.mark.parametrize("route", ["fp16", "int8", None])
def test_first_row_attends_only_to_first_key(oracle_mod, route):
    w = wl.custom(route=route, seed=6, **SHAPES[1])
    out = run_oracle(oracle_mod, w)[0]
    cu = w.cu_seqlens
    for b in range(w.batch):
        if w.seqlens[b] == 0:
            continue
        for h in range(w.hq):
            np.testing.assert_array_equal(out[cu[b], h],
                                          w.v[cu[b], h // (w.hq // w.hk)].astype(np.float32))


def test_route_bit_selects_tile_group(oracle_mod):
    """With Q exactly representable by its own INT8 quantization (Q = delta_q q8), an INT8-routed
    group scores Q . K_hat_j and an FP16 group scores Q . K_j. The routed result is therefore
    textbook attention on K' with K'_j = K_hat_j exactly where the expanded route map says INT8.
    This pins the row (query tile) and column (key tile group) indexing of the route map."""
    shape = dict(seqlens=[150, 70], hq=4, hk=2, d=32, bm_r=32, bn_r=16, group=2, causal=True)
    w = wl.custom(p_fp16=0.5, seed=8, **shape)
    rng = np.random.default_rng(9)
    ints = rng.integers(-127, 128, size=w.q.shape)
    ints[..., 0] = 127  # make every row's max exactly 127 * delta
    delta = 2.0 ** rng.integers(-6, -3, size=w.q.shape[:2])
    w.q[:] = (ints * delta[..., None]).astype(np.float16)
    q8, qs = oracle_mod.quantize_rows(w.q)
    assert np.array_equal(dequant(q8, qs), w.q.astype(np.float64))
    out = run_oracle(oracle_mod, w)[0]
    k8, ks = oracle_mod.quantize_rows(w.k)
    khat = dequant(k8, ks)
    k64 = w.k.astype(np.float64)
    cu = w.cu_seqlens
    rep = w.hq // w.hk
    scale = 1 / np.sqrt(w.d)
    for h in range(w.hq):
        maps = expand_route(w.route[h // rep], w.seqlens, w.bm_r, w.bn_r, w.group)
        for b, L in enumerate(w.seqlens):
            E = maps[b]
            qb = w.q[cu[b]:cu[b + 1], h].astype(np.float64)
            kb, khb = k64[cu[b]:cu[b + 1], h // rep], khat[cu[b]:cu[b + 1], h // rep]
            S = np.where(E, qb @ khb.T, qb @ kb.T) * scale
            S = np.where(np.tril(np.ones((L, L), bool)), S, -np.inf)
            P = np.exp(S - S.max(1, keepdims=True))
            ref = (P @ w.v[cu[b]:cu[b + 1], h // rep].astype(np.float64)) / P.sum(1)[:, None]
            np.testing.assert_allclose(out[cu[b]:cu[b + 1], h], ref, rtol=F32, atol=1e-12)
    # and a different map changes the answer (the bits are read at all)
    w2 = wl.custom(p_fp16=0.5, seed=8, **shape)
    w2.q[:] = w.q
    w2.route[:] = 1 - w.route
    assert np.abs(run_oracle(oracle_mod, w2)[0] - out).max() > 1e-4


def online_softmax(S, V, bn):
    """Section 3.1 recurrence over key blocks of width bn (m, z, O), then O / z. -inf = masked."""
    L = S.shape[0]
    m = np.full(L, -np.inf)
    z = np.zeros(L)
    O = np.zeros((L, V.shape[1]))
    for j0 in range(0, S.shape[1], bn):
        Sb = S[:, j0:j0 + bn]
        m_new = np.maximum(m, Sb.max(axis=1))
        safe = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(m - safe), 0.0)
        Pb = np.where(np.isfinite(Sb), np.exp(Sb - safe[:, None]), 0.0)
        z = alpha * z + Pb.sum(axis=1)
        O = alpha[:, None] * O + Pb @ V[j0:j0 + bn]
        m = m_new
    return O / z[:, None]


@pytest.mark.parametrize("bn", [1, 5, 16, 64])
def test_online_recurrence_matches_two_pass_all_masks(oracle_mod, bn):
    """Every mask over T_mask = 4 groups (same pattern in every query-tile row), plus random
    per-row masks, on L = 64, d = 16: the blocked online recurrence equals the two-pass oracle."""
    L, d = 64, 16
    base = wl.custom(seqlens=[L], hq=1, hk=1, d=d, bm_r=16, bn_r=16, group=1, causal=True,
                     route="fp16", seed=10)
    q8, qs = oracle_mod.quantize_rows(base.q)
    k8, ks = oracle_mod.quantize_rows(base.k)
    S16 = (base.q[:, 0].astype(np.float64) @ base.k[:, 0].astype(np.float64).T) / np.sqrt(d)
    S8 = (dequant(q8, qs)[:, 0] @ dequant(k8, ks)[:, 0].T) / np.sqrt(d)
    causal = np.tril(np.ones((L, L), bool))
    patterns = [np.array(bits, dtype=np.uint8) for bits in itertools.product([0, 1], repeat=4)]
    rng = np.random.default_rng(11)
    maps = [np.tile(p, (4, 1)) for p in patterns] + [(rng.random((4, 4)) < 0.5).astype(np.uint8)
                                                    for _ in range(8)]
    for R in maps:
        base.route[0] = R
        out = run_oracle(oracle_mod, base)[0][:, 0]
        E = expand_route(R, [L], 16, 16, 1)[0]
        S = np.where(causal, np.where(E, S8, S16), -np.inf)
        ref = online_softmax(S, base.v[:, 0].astype(np.float64), bn)
        np.testing.assert_allclose(out, ref, rtol=F32, atol=1e-12)


def test_gqa_equals_repeated_kv_heads(oracle_mod):
    w = wl.custom(seqlens=[90, 33], hq=6, hk=2, d=32, bm_r=16, bn_r=16, group=1, seed=12)
    out = run_oracle(oracle_mod, w)[0]
    rep = w.hq // w.hk
    w2 = wl.custom(seqlens=[90, 33], hq=6, hk=6, d=32, bm_r=16, bn_r=16, group=1, seed=12)
    w2.q[:] = w.q
    w2.k = np.repeat(w.k, rep, axis=1)
    w2.v = np.repeat(w.v, rep, axis=1)
    w2.route = np.repeat(w.route, rep, axis=0)
    out2 = run_oracle(oracle_mod, w2)[0]
    np.testing.assert_array_equal(out, out2)


def test_varlen_equals_separate_sequences(oracle_mod):
    lens = [45, 0, 100, 17]
    w = wl.custom(seqlens=lens, hq=4, hk=2, d=32, bm_r=16, bn_r=16, group=2, seed=13)
    out = run_oracle(oracle_mod, w)[0]
    cu, cm = w.cu_seqlens, w.cu_mtiles
    for b, L in enumerate(lens):
        if L == 0:
            continue
        wb = wl.custom(seqlens=[L], hq=4, hk=2, d=32, bm_r=16, bn_r=16, group=2, seed=13)
        wb.q, wb.k, wb.v = (x[cu[b]:cu[b + 1]].copy() for x in (w.q, w.k, w.v))
        tb = -(-L // (16 * 2))
        wb.route = w.route[:, cm[b]:cm[b + 1], :tb].copy()
        np.testing.assert_array_equal(run_oracle(oracle_mod, wb)[0], out[cu[b]:cu[b + 1]])


@pytest.mark.parametrize("g", [2, 3])
def test_grouping_equals_repeated_bits(oracle_mod, g):
    """Section 4.2 grouping: a group-g map equals the group-1 map with each bit repeated g times."""
    w = wl.custom(seqlens=[200], hq=2, hk=1, d=32, bm_r=32, bn_r=16, group=g, seed=14)
    out = run_oracle(oracle_mod, w)[0]
    w1 = wl.custom(seqlens=[200], hq=2, hk=1, d=32, bm_r=32, bn_r=16, group=1, seed=14)
    w1.q, w1.k, w1.v = w.q, w.k, w.v
    n1 = w1.route.shape[2]
    w1.route = np.repeat(w.route, g, axis=2)[:, :, :n1].copy()
    np.testing.assert_array_equal(run_oracle(oracle_mod, w1)[0], out)


def test_bottom_right_causal_with_unequal_lengths(oracle_mod):
    """L_q < L_k: query i sees keys j <= i + (L_k - L_q) (all-FP16 and all-INT8 maps)."""
    rng = np.random.default_rng(15)
    Lq, Lk, hq, hk, d, bm, bn = 40, 100, 2, 1, 32, 16, 16
    q = rng.standard_normal((Lq, hq, d)).astype(np.float16)
    k = rng.standard_normal((Lk, hk, d)).astype(np.float16)
    v = rng.standard_normal((Lk, hk, d)).astype(np.float16)
    cu_q, cu_k = np.array([0, Lq]), np.array([0, Lk])
    cu_m = np.array([0, -(-Lq // bm)])
    q8, qs = oracle_mod.quantize_rows(q)
    k8, ks = oracle_mod.quantize_rows(k)
    for bit in (0, 1):
        R = np.full((hk, cu_m[-1], -(-Lk // bn)), bit, np.uint8)
        prep = oracle_mod.Prepared(q=q, k=k, v=v, cu_q=cu_q, cu_k=cu_k, cu_mtiles=cu_m, hq=hq,
                                   hk=hk, d=d, words=oracle_mod.pack_route(R), bm_r=bm, bn_r=bn,
                                   group=1, causal=True, q8=q8, q_scale=qs, k8=k8, k_scale=ks)
        out = prep.prefill()[0]
        qq = dequant(q8, qs) if bit else q
        kk = dequant(k8, ks) if bit else k
        ref, _ = textbook(qq, kk, v, cu_q, cu_k, hq, hk, True)
        np.testing.assert_allclose(out, ref, rtol=F32, atol=1e-12)


def test_kv_int8_cache_is_attention_on_dequantized_cache(oracle_mod):
    """INT8 K/V cache: FP16 tiles use K = delta_k k8, P.V uses V = delta_v v8; INT8 tiles use
    delta_q delta_k (q8 . k8)."""
    for route in ("fp16", "int8"):
        w = wl.custom(seqlens=[100, 60], hq=4, hk=2, d=64, bm_r=32, bn_r=32, group=1,
                      route=route, kv_int8=True, seed=16)
        out = run_oracle(oracle_mod, w)[0]
        q8, qs = oracle_mod.quantize_rows(w.q)
        k8, ks = oracle_mod.quantize_rows(w.k)
        v8, vs = oracle_mod.quantize_rows(w.v)
        qq = dequant(q8, qs) if route == "int8" else w.q
        ref, _ = textbook(qq, dequant(k8, ks), dequant(v8, vs), w.cu_seqlens, w.cu_seqlens,
                          w.hq, w.hk, True)
        np.testing.assert_allclose(out, ref, rtol=F32, atol=1e-12)


def test_row_sampling_matches_full_run(oracle_mod):
    w = wl.custom(seqlens=[100, 60], hq=4, hk=2, d=32, bm_r=32, bn_r=16, group=2, seed=17)
    prep = oracle_mod.prepare(w)
    full, full_lse, _, _ = prep.prefill()
    rows = np.array([0, 5, 99, 100, 159, 42])
    part, part_lse, _, _ = prep.prefill(rows)
    np.testing.assert_array_equal(part, full[rows])
    np.testing.assert_array_equal(part_lse, full_lse[:, rows])


def test_int32_tiles_are_exact_integer_products(oracle_mod):
    w = wl.custom(seqlens=[100, 70], hq=4, hk=2, d=64, bm_r=32, bn_r=32, group=1, p_fp16=0.4,
                  seed=18)
    prep = oracle_mod.prepare(w)
    q8, _ = oracle_mod.quantize_rows(w.q)
    k8, _ = oracle_mod.quantize_rows(w.k)
    head, hk = 3, 3 // 2
    ntiles = 4
    fill = np.iinfo(np.int32).min
    dump = prep.int32_tiles(head, 0, w.total_mtiles, ntiles, fill=fill)
    cu, cm = w.cu_seqlens, w.cu_mtiles
    bound = w.d * 127 * 127
    for b, L in enumerate(w.seqlens):
        acc = q8[cu[b]:cu[b + 1], head].astype(np.int64) @ k8[cu[b]:cu[b + 1], hk].astype(np.int64).T
        assert np.abs(acc).max() <= bound
        for m in range(cm[b + 1] - cm[b]):
            r = cm[b] + m
            for n in range(ntiles):
                tile = dump[r, n]
                i0, j0 = m * 32, n * 32
                inb = (min(L, i0 + 32) - i0, max(0, min(L, j0 + 32) - j0))
                legal = j0 <= min(L, i0 + 32) - 1 and inb[1] > 0
                if w.route[hk, r, n] and legal:
                    np.testing.assert_array_equal(tile[:inb[0], :inb[1]],
                                                  acc[i0:i0 + inb[0], j0:j0 + inb[1]])
                    assert np.all(tile[inb[0]:] == fill) and np.all(tile[:, inb[1]:] == fill)
                else:
                    assert np.all(tile == fill)


def test_named_workload_metadata():
    s, L = wl.varlen_lengths()
    assert s == 3 and sum(L) == 65752
    w = wl.make("tiny")
    assert w.route.shape == (2, 4, 4) and w.words_per_row == 1
    assert w.legal_pairs() == 256 * 257 // 2
