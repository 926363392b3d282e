"""Seeded synthetic inputs for routed prefill attention.

This module only draws inputs: fp16 Q/K/V in the packed varlen layout ``[tokens, heads, d]``,
the sequence metadata (``cu_seqlens``, ``cu_mtiles``) and a uint8 routing map
``R[h_k, route_row, g_j]`` (1 = INT8 score path, 0 = FP16 score path, as in Section 4.2 of the
TileMix paper). It holds none of the attention or quantization arithmetic; both the HIP path and
the CPU oracle take their inputs from here.

The five named workloads mirror the shapes of the paper's prefill settings (LLaMA/Qwen-like head
counts, GQA, varlen batches, long contexts, an INT8 K/V cache). The paper's own evaluation data
(LongEval, LV-Eval and model activations) are not available, so i.i.d. standard-normal
activations stand in for them, with heavy-tailed outlier channels in K where a workload asks
for them.

Draw order for a seed: Q, K, V (float32 standard normal, layout [T, H, d]), then the
workload's extras (outlier channels), then the fp16 cast, then the routing map.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

__all__ = ["Workload", "make", "custom", "WORKLOADS", "varlen_lengths", "DecodeWorkload",
           "make_decode", "decode_custom", "DECODE_WORKLOADS", "numerics_case", "NUMERICS_LENGTHS",
           "NUMERICS_COVERAGES"]


@dataclasses.dataclass
class Workload:
    name: str
    hq: int
    hk: int
    d: int
    seqlens: List[int]
    causal: bool
    bm_r: int           # route tile rows (query tokens per routing row)
    bn_r: int           # route tile columns (key tokens per key tile)
    group: int          # key tiles per routing bit (grouping factor g)
    kv_int8: bool       # K/V arrive as an INT8 cache (quantized by the consumer's own quantizer)
    q: np.ndarray       # fp16 [T, hq, d]
    k: np.ndarray       # fp16 [T, hk, d]
    v: np.ndarray       # fp16 [T, hk, d]
    route: np.ndarray   # uint8 [hk, total_mtiles, t_mask]
    policy: str = ""
    seed: int = 0

    @property
    def batch(self) -> int:
        return len(self.seqlens)

    @property
    def total(self) -> int:
        return int(sum(self.seqlens))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)

    @property
    def cu_mtiles(self) -> np.ndarray:
        tiles = [-(-L // self.bm_r) for L in self.seqlens]
        return np.concatenate([[0], np.cumsum(tiles)]).astype(np.int32)

    @property
    def total_mtiles(self) -> int:
        return int(self.cu_mtiles[-1])

    @property
    def t_mask(self) -> int:
        return int(self.route.shape[2])

    @property
    def words_per_row(self) -> int:
        return max(1, -(-self.t_mask // 64))

    def legal_pairs(self) -> int:
        """Legal (query, key) pairs per query head (causal: L(L+1)/2 per sequence)."""
        if self.causal:
            return int(sum(L * (L + 1) // 2 for L in self.seqlens))
        return int(sum(L * L for L in self.seqlens))

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "batch": self.batch,
            "seqlens": self.seqlens if len(self.seqlens) <= 16 else f"{len(self.seqlens)} seqs",
            "total_tokens": self.total,
            "hq": self.hq,
            "hk": self.hk,
            "head_dim": self.d,
            "causal": self.causal,
            "route_tile": [self.bm_r, self.bn_r],
            "group": self.group,
            "t_mask": self.t_mask,
            "kv_int8": self.kv_int8,
            "policy": self.policy,
            "seed": self.seed,
        }


def varlen_lengths(n: int = 8, lo: int = 1024, hi: int = 16384, total_lo: int = 60_000,
                   total_hi: int = 68_000) -> tuple:
    """Lengths uniform in [lo, hi] from the first seed >= 0 whose total lies in [total_lo, total_hi]."""
    for s in range(10_000):
        L = np.random.default_rng(s).integers(lo, hi + 1, n)
        if total_lo <= int(L.sum()) <= total_hi:
            return s, [int(x) for x in L]
    raise RuntimeError("no seed gives the requested total")


def _draw_qkv(rng, T, hq, hk, d):
    q = rng.standard_normal((T, hq, d), dtype=np.float32)
    k = rng.standard_normal((T, hk, d), dtype=np.float32)
    v = rng.standard_normal((T, hk, d), dtype=np.float32)
    return q, k, v


def _geometry(seqlens, bm_r, bn_r, group):
    total_mtiles = sum(-(-L // bm_r) for L in seqlens)
    t_mask = max(1, max(-(-L // (bn_r * group)) for L in seqlens))
    return total_mtiles, t_mask


def _group_valid(seqlens, bm_r, bn_r, group, t_mask):
    """valid[row, g] = group g exists for the sequence that route row belongs to."""
    rows = []
    for L in seqlens:
        ng = -(-L // (bn_r * group))
        row = np.zeros(t_mask, dtype=bool)
        row[:ng] = True
        rows += [row] * (-(-L // bm_r))
    return np.stack(rows) if rows else np.zeros((0, t_mask), dtype=bool)


def route_bernoulli(rng, hk, seqlens, bm_r, bn_r, group, p_fp16):
    total_mtiles, t_mask = _geometry(seqlens, bm_r, bn_r, group)
    fp16 = rng.random((hk, total_mtiles, t_mask)) < p_fp16
    r = (~fp16).astype(np.uint8)
    r &= _group_valid(seqlens, bm_r, bn_r, group, t_mask)[None].astype(np.uint8)
    return r


def route_constant(hk, seqlens, bm_r, bn_r, group, bit):
    total_mtiles, t_mask = _geometry(seqlens, bm_r, bn_r, group)
    r = np.full((hk, total_mtiles, t_mask), bit, dtype=np.uint8)
    r &= _group_valid(seqlens, bm_r, bn_r, group, t_mask)[None].astype(np.uint8)
    return r


def route_topk_maxabs(k16: np.ndarray, seqlens, bm_r, bn_r, group, frac_fp16):
    """Per KV head, the ceil(frac * T_mask) key groups with the largest max|K| are FP16 in every row.

    Single-sequence policy (ties go to the lower group index)."""
    assert len(seqlens) == 1
    L = seqlens[0]
    total_mtiles, t_mask = _geometry(seqlens, bm_r, bn_r, group)
    span = bn_r * group
    hk = k16.shape[1]
    nsel = int(math.ceil(frac_fp16 * t_mask - 1e-9))
    r = np.ones((hk, total_mtiles, t_mask), dtype=np.uint8)
    for h in range(hk):
        gmax = np.array([np.abs(k16[g * span:min((g + 1) * span, L), h, :].astype(np.float32)).max()
                         for g in range(t_mask)])
        order = np.lexsort((np.arange(t_mask), -gmax))  # descending max, ascending index on ties
        r[h, :, order[:nsel]] = 0
    return r


def make(name: str, seed: int = 0) -> Workload:
    """The named synthetic workloads (shapes of the paper's prefill settings)."""
    rng = np.random.default_rng(seed)
    if name == "tiny":
        seqlens, hq, hk, d = [256], 2, 2, 64
        bm_r, bn_r, g = 64, 64, 1
        q, k, v = _draw_qkv(rng, 256, hq, hk, d)
        q, k, v = (x.astype(np.float16) for x in (q, k, v))
        route = route_bernoulli(rng, hk, seqlens, bm_r, bn_r, g, 0.5)
        return Workload(name, hq, hk, d, seqlens, True, bm_r, bn_r, g, False, q, k, v, route,
                        "bernoulli(p_fp16=0.5)", seed)
    if name == "mha8k":
        seqlens, hq, hk, d = [8192], 32, 32, 128
        bm_r, bn_r, g = 128, 128, 1
        q, k, v = _draw_qkv(rng, 8192, hq, hk, d)
        q, k, v = (x.astype(np.float16) for x in (q, k, v))
        route = route_bernoulli(rng, hk, seqlens, bm_r, bn_r, g, 0.25)
        return Workload(name, hq, hk, d, seqlens, True, bm_r, bn_r, g, False, q, k, v, route,
                        "bernoulli(p_fp16=0.25)", seed)
    if name == "gqa32k":
        seqlens, hq, hk, d = [32768], 32, 8, 128
        bm_r, bn_r, g = 128, 128, 4
        q, k, v = _draw_qkv(rng, 32768, hq, hk, d)
        for h in range(hk):
            ch = rng.choice(d, 4, replace=False)
            k[:, h, ch] *= 20.0
        q, k, v = (x.astype(np.float16) for x in (q, k, v))
        route = route_topk_maxabs(k, seqlens, bm_r, bn_r, g, 0.10)
        return Workload(name, hq, hk, d, seqlens, True, bm_r, bn_r, g, False, q, k, v, route,
                        "top-10% max|K| groups FP16 (4 outlier channels x20 per KV head)", seed)
    if name == "varlen64k":
        _, seqlens = varlen_lengths()
        hq, hk, d = 28, 4, 128
        bm_r, bn_r, g = 128, 128, 2
        T = sum(seqlens)
        q, k, v = _draw_qkv(rng, T, hq, hk, d)
        q, k, v = (x.astype(np.float16) for x in (q, k, v))
        route = route_bernoulli(rng, hk, seqlens, bm_r, bn_r, g, 0.20)
        return Workload(name, hq, hk, d, seqlens, True, bm_r, bn_r, g, False, q, k, v, route,
                        "bernoulli(p_fp16=0.20)", seed)
    if name == "kvint8_128k":
        seqlens, hq, hk, d = [131072], 32, 8, 128
        bm_r, bn_r, g = 128, 128, 8
        q, k, v = _draw_qkv(rng, 131072, hq, hk, d)
        q, k, v = (x.astype(np.float16) for x in (q, k, v))
        route = route_bernoulli(rng, hk, seqlens, bm_r, bn_r, g, 0.05)
        return Workload(name, hq, hk, d, seqlens, True, bm_r, bn_r, g, True, q, k, v, route,
                        "bernoulli(p_fp16=0.05); K/V as INT8 cache", seed)
    raise KeyError(f"unknown workload {name!r}; known: {WORKLOADS}")


WORKLOADS = ("tiny", "mha8k", "gqa32k", "varlen64k", "kvint8_128k")


def custom(seqlens: Sequence[int], hq: int, hk: int, d: int, *, causal: bool = True,
           bm_r: int = 64, bn_r: int = 64, group: int = 1, p_fp16: float = 0.5,
           route: Optional[str] = None, kv_int8: bool = False, seed: int = 0,
           q_std: float = 1.0, k_std: float = 1.0, name: str = "custom") -> Workload:
    """A small workload for tests: route = None (Bernoulli p_fp16), "int8" (all 1) or "fp16" (all 0)."""
    rng = np.random.default_rng(seed)
    T = int(sum(seqlens))
    q, k, v = _draw_qkv(rng, T, hq, hk, d)
    q *= q_std
    k *= k_std
    q, k, v = (x.astype(np.float16) for x in (q, k, v))
    seqlens = [int(x) for x in seqlens]
    if route is None:
        r = route_bernoulli(rng, hk, seqlens, bm_r, bn_r, group, p_fp16)
        pol = f"bernoulli(p_fp16={p_fp16})"
    elif route == "int8":
        r = route_constant(hk, seqlens, bm_r, bn_r, group, 1)
        pol = "all INT8"
    elif route == "fp16":
        r = route_constant(hk, seqlens, bm_r, bn_r, group, 0)
        pol = "all FP16"
    else:
        raise ValueError(route)
    return Workload(name, hq, hk, d, seqlens, causal, bm_r, bn_r, group, kv_int8, q, k, v, r,
                    pol, seed)



# ----------------------------------------------------------------------------- numerics sweep

NUMERICS_LENGTHS = (1024, 2048, 4096, 8192)
NUMERICS_COVERAGES = (0.0, 0.05, 0.10, 0.15, 0.20, 0.25)


def numerics_case(L: int, int8_coverage: float, seed: int = 0) -> Workload:
    """Randomized attention inputs for the output-deviation sweep over INT8 tile-group coverage
    (the setting of the TileMix paper's Section 5.4 / Table 3): one causal sequence of L tokens,
    24 query / 8 KV heads of 128 channels (the head layout of the 3B model the paper times),
    64 x 64 route tiles, one tile per routing bit, each group INT8 with probability
    int8_coverage. Inputs do not depend on the coverage, only the route map does."""
    rng = np.random.default_rng(seed)
    hq, hk, d, bm_r, bn_r, g = 24, 8, 128, 64, 64, 1
    q, k, v = _draw_qkv(rng, L, hq, hk, d)
    q, k, v = (x.astype(np.float16) for x in (q, k, v))
    rrng = np.random.default_rng([seed, int(round(int8_coverage * 10000))])
    route = route_bernoulli(rrng, hk, [L], bm_r, bn_r, g, 1.0 - int8_coverage)
    return Workload(f"numerics_L{L}_int8_{int(round(100 * int8_coverage))}pct", hq, hk, d, [L], True,
                    bm_r, bn_r, g, False, q, k, v, route,
                    f"bernoulli(int8_coverage={int8_coverage})", seed)

# ----------------------------------------------------------------------------- decode

@dataclasses.dataclass
class DecodeWorkload:
    """A few new query tokens per sequence against a cached K/V of L_k tokens (the new tokens are
    the cache's last L_q positions, so causal alignment is bottom-right). K and V are drawn in
    fp16; the consumer quantizes them into its INT8 cache with its own quantizer."""
    name: str
    hq: int
    hk: int
    d: int
    q_lens: List[int]       # L_q per sequence (new tokens)
    k_lens: List[int]       # L_k per sequence (cached tokens, the new ones included)
    causal: bool
    bm_r: int
    bn_r: int
    group: int
    q: np.ndarray           # fp16 [sum L_q, hq, d]
    k: np.ndarray           # fp16 [sum L_k, hk, d]
    v: np.ndarray           # fp16 [sum L_k, hk, d]
    route: np.ndarray       # uint8 [hk, total_mtiles, t_mask]
    policy: str = ""
    seed: int = 0
    kv_int8: bool = True

    @property
    def batch(self) -> int:
        return len(self.q_lens)

    @property
    def total_q(self) -> int:
        return int(sum(self.q_lens))

    @property
    def total_k(self) -> int:
        return int(sum(self.k_lens))

    @property
    def cu_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    @property
    def cu_k(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.k_lens)]).astype(np.int32)

    @property
    def cu_mtiles(self) -> np.ndarray:
        tiles = [-(-L // self.bm_r) for L in self.q_lens]
        return np.concatenate([[0], np.cumsum(tiles)]).astype(np.int32)

    @property
    def t_mask(self) -> int:
        return int(self.route.shape[2])

    @property
    def words_per_row(self) -> int:
        return max(1, -(-self.t_mask // 64))

    def legal_pairs(self) -> int:
        """Legal (query, key) pairs per query head."""
        n = 0
        for lq, lk in zip(self.q_lens, self.k_lens):
            for i in range(lq):
                n += min(lk, i + lk - lq + 1) if self.causal else lk
        return n

    def describe(self) -> dict:
        return {"workload": self.name, "batch": self.batch,
                "q_lens": self.q_lens if self.batch <= 16 else f"{self.batch} seqs",
                "k_lens": self.k_lens if self.batch <= 16 else f"{self.batch} seqs",
                "hq": self.hq, "hk": self.hk, "head_dim": self.d, "causal": self.causal,
                "route_tile": [self.bm_r, self.bn_r], "group": self.group, "t_mask": self.t_mask,
                "kv_int8": True, "policy": self.policy, "seed": self.seed}


def decode_custom(q_lens: Sequence[int], k_lens: Sequence[int], hq: int, hk: int, d: int, *,
                  causal: bool = True, bm_r: int = 128, bn_r: int = 128, group: int = 1,
                  p_fp16: float = 0.5, route: Optional[str] = None, seed: int = 0,
                  k_std: float = 1.0, name: str = "decode") -> DecodeWorkload:
    """Draw order: Q [sum L_q], K, V [sum L_k] (standard normal), the fp16 cast, then the route
    map (Bernoulli p_fp16, or constant "int8" / "fp16"), one route row per query tile."""
    rng = np.random.default_rng(seed)
    q_lens, k_lens = [int(x) for x in q_lens], [int(x) for x in k_lens]
    Tq, Tk = sum(q_lens), sum(k_lens)
    q = rng.standard_normal((Tq, hq, d), dtype=np.float32)
    k = rng.standard_normal((Tk, hk, d), dtype=np.float32) * k_std
    v = rng.standard_normal((Tk, hk, d), dtype=np.float32)
    q, k, v = (x.astype(np.float16) for x in (q, k, v))
    rows = sum(-(-L // bm_r) for L in q_lens)
    t_mask = max(1, max(-(-L // (bn_r * group)) for L in k_lens))
    valid = []
    for lq, lk in zip(q_lens, k_lens):
        row = np.zeros(t_mask, dtype=bool)
        row[:-(-lk // (bn_r * group))] = True
        valid += [row] * (-(-lq // bm_r))
    valid = np.stack(valid) if valid else np.zeros((0, t_mask), dtype=bool)
    if route is None:
        r = (rng.random((hk, rows, t_mask)) >= p_fp16).astype(np.uint8)
        pol = f"bernoulli(p_fp16={p_fp16})"
    else:
        r = np.full((hk, rows, t_mask), 1 if route == "int8" else 0, dtype=np.uint8)
        pol = "all INT8" if route == "int8" else "all FP16"
    r &= valid[None].astype(np.uint8)
    return DecodeWorkload(name, hq, hk, d, q_lens, k_lens, causal, bm_r, bn_r, group, q, k, v, r,
                          pol, seed)


def make_decode(name: str, seed: int = 0) -> DecodeWorkload:
    """Named decode workloads: one new token against the 128k INT8 cache of the long-prefill
    setting (32 query / 8 KV heads, route group 8, 5 % FP16 groups), and a varlen batch."""
    if name == "decode128k":
        return decode_custom([1], [131072], 32, 8, 128, bm_r=128, bn_r=128, group=8, p_fp16=0.05,
                             seed=seed, name=name)
    if name == "decode_batch":
        return decode_custom([1, 1, 2, 4, 1, 1, 3, 1], [16384, 9000, 4096, 30000, 777, 2048, 12345, 64],
                             32, 8, 128, bm_r=128, bn_r=128, group=2, p_fp16=0.2, seed=seed, name=name)
    raise KeyError(name)


DECODE_WORKLOADS = ("decode128k", "decode_batch")

