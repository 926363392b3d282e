"""Pins of the oracle's block-wise quantizer (one scale per block of tokens of one sequence and
head; TileMix paper, Section 4.3 "blockwise ... per-block scales", quantizer psi of Section
3.2): hand-worked cases, the rounding bound |delta * code - x| <= delta / 2, the shared scale and
the full code range of every block, block independence across sequence boundaries, and the
one-token-block case against the per-token quantizer."""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def built():
    oracle.build()


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def test_block_golden_cases():
    cases = json.load(open(os.path.join(GOLDEN, "quantize_block_cases.json")))["cases"]
    for c in cases:
        x = np.array(c["rows"], dtype=np.float16)[:, None, :]
        q, s = oracle.quantize_blocks(x, _cu(c["seqlens"]), c["block_rows"])
        assert q[:, 0, :].tolist() == c["q"], c["why"]


def test_block_scale_value():
    x = np.array([[1, 2, 3, 4], [-8, 0.5, 2, -1]], dtype=np.float16)[:, None, :]
    _, s = oracle.quantize_blocks(x, _cu([2]), 2)
    assert s[0, 0] == s[1, 0] == np.float32(8.0) / np.float32(127.0)


@pytest.mark.parametrize("block", [1, 7, 64, 128, 5000])
def test_block_invariants(block):
    rng = np.random.default_rng(block)
    lens = [300, 1, 0, 777, 128]
    T, H, d = sum(lens), 3, 64
    x = (rng.standard_normal((T, H, d)) * rng.uniform(0.01, 50, (T, H, 1))).astype(np.float16)
    x[5:9] = 0
    q, s = oracle.quantize_blocks(x, _cu(lens), block)
    xf = x.astype(np.float64)
    # rounding bound of every element: |delta q - x| <= delta |q - x inv| + |x| |delta inv - 1|
    # <= delta (1/2 + ulp(x inv) + 127 * 2^-22), with inv = fl(127 / a), delta = fl(a / 127)
    d64 = s[:, :, None].astype(np.float64)
    assert np.all(np.abs(d64 * q - xf) <= d64 * (0.5 + 2.0**-17 + 127 * 2.0**-22))
    cu = _cu(lens)
    for b in range(len(lens)):
        for t0 in range(cu[b], cu[b + 1], block):
            t1 = min(cu[b + 1], t0 + block)
            for h in range(H):
                blk = s[t0:t1, h]
                assert np.all(blk == blk[0])  # one scale per block
                a = np.abs(xf[t0:t1, h]).max()
                if a == 0:
                    assert blk[0] == 0 and not q[t0:t1, h].any()
                else:
                    assert np.abs(q[t0:t1, h]).max() == 127  # the block max maps to +-127
                    assert abs(blk[0] * 127 - a) <= a * 2e-7


def test_blocks_do_not_straddle_sequences():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((200, 2, 64)).astype(np.float16)
    q1, s1 = oracle.quantize_blocks(x[:100], _cu([100]), 64)
    y = x.copy()
    y[100:] *= 1000  # huge values in the second sequence only
    q2, s2 = oracle.quantize_blocks(y, _cu([100, 100]), 64)
    assert np.array_equal(q1, q2[:100]) and np.array_equal(s1, s2[:100])


def test_one_token_blocks_equal_per_token_quantizer():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 4, 128)).astype(np.float16)
    qb, sb = oracle.quantize_blocks(x, _cu([20, 30]), 1)
    qr, sr = oracle.quantize_rows(x)
    assert np.array_equal(qb, qr) and np.array_equal(sb, sr)
