"""TEST INFRASTRUCTURE ONLY: ctypes front end of the CPU oracle (``tilemix_oracle.cpp``).

Only the test suite, the package smoke check and the benchmark's CPU-baseline leg may import
this package. The product path (the HIP library and its binding) never does.

The oracle is a plain, slow, fp64 implementation of tile-group precision-routed attention as
defined in "TileMix: Tile-Centric Mixed-Precision Attention for LLM Inference Acceleration"
(Sections 3.1, 3.2, 4.1-4.3). See the header of ``tilemix_oracle.cpp`` for the exact readings.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tilemix_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with g++ (-O3, OpenMP, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["g++", "-O3", "-std=c++17", "-fopenmp", "-fPIC", "-shared",
                               "-ffp-contract=off", "-fno-fast-math", "-o", tmp, _SRC])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("hq", ctypes.c_int32), ("hk", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("total_q", ctypes.c_int64), ("total_k", ctypes.c_int64),
        ("cu_q", ctypes.c_void_p), ("cu_k", ctypes.c_void_p), ("cu_mtiles", ctypes.c_void_p),
        ("total_mtiles", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("q8", ctypes.c_void_p), ("q_scale", ctypes.c_void_p),
        ("k8", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
        ("v8", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("kv_int8", ctypes.c_int32),
        ("words", ctypes.c_void_p),
        ("wpr", ctypes.c_int32), ("bm_r", ctypes.c_int32), ("bn_r", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("softmax_scale", ctypes.c_double),
    ]


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_quantize_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                           ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_quantize_blocks.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_pack_route.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_int32]
        L.oracle_prefill.argtypes = [ctypes.POINTER(Problem), ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]
        L.oracle_int32_tiles.argtypes = [ctypes.POINTER(Problem), ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        L.oracle_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_philox4x32_10.restype = None
        L.oracle_route_topk_maxabs.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        L.oracle_route_bernoulli.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p]
        L.oracle_decode_fp16.argtypes = [ctypes.c_uint16]
        L.oracle_decode_fp16.restype = ctypes.c_double
        _lib = L
    return _lib


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def decode_fp16(bits: int) -> float:
    return float(lib().oracle_decode_fp16(int(bits)))


def quantize_rows(x: np.ndarray):
    """Per-row symmetric INT8 of an fp16 array [..., d] -> (int8 [..., d], fp32 scale [...])."""
    x = np.ascontiguousarray(x, dtype=np.float16)
    d = x.shape[-1]
    rows = x.size // d
    q = np.empty(x.shape, dtype=np.int8)
    s = np.empty(x.shape[:-1], dtype=np.float32)
    rc = lib().oracle_quantize_rows(_ptr(x), rows, d, d, _ptr(q), _ptr(s))
    if rc:
        raise ValueError("oracle_quantize_rows rejected its arguments")
    return q, s


def quantize_blocks(x: np.ndarray, cu_seqlens, block_rows: int):
    """Block-wise symmetric INT8 of fp16 [T, H, d]: one scale per (block of block_rows tokens of a
    sequence, head), repeated on each row -> (int8 [T, H, d], fp32 scale [T, H])."""
    x = np.ascontiguousarray(x, dtype=np.float16)
    T, H, d = x.shape
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    q = np.empty(x.shape, dtype=np.int8)
    s = np.empty((T, H), dtype=np.float32)
    rc = lib().oracle_quantize_blocks(_ptr(x.view(np.uint16)), T, H, d, _ptr(cu), len(cu) - 1,
                                      block_rows, _ptr(q), _ptr(s))
    if rc:
        raise ValueError("oracle_quantize_blocks rejected its arguments")
    return q, s


def pack_route(route: np.ndarray, wpr: Optional[int] = None) -> np.ndarray:
    """uint8 R [..., t_mask] of 0/1 -> uint64 words [..., wpr] (bit g_j = word g_j>>6, bit g_j&63)."""
    route = np.ascontiguousarray(route, dtype=np.uint8)
    t_mask = route.shape[-1]
    wpr = wpr or max(1, -(-t_mask // 64))
    rows = route.size // t_mask if t_mask else int(np.prod(route.shape[:-1]))
    words = np.empty(route.shape[:-1] + (wpr,), dtype=np.uint64)
    rc = lib().oracle_pack_route(_ptr(route), rows, t_mask, _ptr(words), wpr)
    if rc:
        raise ValueError("oracle_pack_route rejected its arguments")
    return words


def philox4x32_10(ctr, key) -> np.ndarray:
    """Philox4x32-10 of a 4-word counter and a 2-word key -> 4 uint32 words."""
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.empty(4, dtype=np.uint32)
    lib().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def _route_geometry(cu_k, cu_mtiles, bn_r, group, t_mask):
    cu_k = np.ascontiguousarray(cu_k, dtype=np.int32)
    cu_mtiles = np.ascontiguousarray(cu_mtiles, dtype=np.int32)
    span = bn_r * group
    if t_mask is None:
        t_mask = max(1, int(max(-(-int(n) // span) for n in np.diff(cu_k))))
    return cu_k, cu_mtiles, int(t_mask)


def route_topk_maxabs(cu_k, cu_mtiles, hk, d, bn_r, group, per_mille, *, k=None, k8=None,
                      k_scale=None, t_mask=None) -> np.ndarray:
    """Top-k by max|K| routing map R [hk, total_mtiles, t_mask] (uint8, 1 = INT8).

    k: fp16 [total_k, hk, d]; or k8 int8 [total_k, hk, d] with k_scale fp32 [total_k, hk]."""
    cu_k, cu_mtiles, t_mask = _route_geometry(cu_k, cu_mtiles, bn_r, group, t_mask)
    kb = None if k is None else np.ascontiguousarray(k, dtype=np.float16).view(np.uint16)
    k8 = None if k8 is None else np.ascontiguousarray(k8, dtype=np.int8)
    ks = None if k_scale is None else np.ascontiguousarray(k_scale, dtype=np.float32)
    R = np.empty((hk, int(cu_mtiles[-1]), t_mask), dtype=np.uint8)
    rc = lib().oracle_route_topk_maxabs(_ptr(cu_k), _ptr(cu_mtiles), len(cu_k) - 1, hk, d, _ptr(kb),
                                        _ptr(k8), _ptr(ks), bn_r, group, per_mille, t_mask, _ptr(R))
    if rc:
        raise ValueError("oracle_route_topk_maxabs rejected its arguments")
    return R


def route_bernoulli(cu_k, cu_mtiles, hk, bn_r, group, per_mille, seed, *, t_mask=None) -> np.ndarray:
    """Coverage-budget Bernoulli routing map R [hk, total_mtiles, t_mask] (uint8, 1 = INT8)."""
    cu_k, cu_mtiles, t_mask = _route_geometry(cu_k, cu_mtiles, bn_r, group, t_mask)
    R = np.empty((hk, int(cu_mtiles[-1]), t_mask), dtype=np.uint8)
    rc = lib().oracle_route_bernoulli(_ptr(cu_k), _ptr(cu_mtiles), len(cu_k) - 1, hk, bn_r, group,
                                      per_mille, int(seed), t_mask, _ptr(R))
    if rc:
        raise ValueError("oracle_route_bernoulli rejected its arguments")
    return R


class Prepared:
    """Holds the arrays of one oracle problem alive for the duration of the calls."""

    def __init__(self, *, q, k, v, cu_q, cu_k, cu_mtiles, hq, hk, d, words, bm_r, bn_r, group,
                 causal, q8, q_scale, k8, k_scale, v8=None, v_scale=None, kv_int8=False,
                 softmax_scale=0.0):
        c = np.ascontiguousarray
        self.arrays = dict(
            q=None if q is None else c(q, dtype=np.float16).view(np.uint16),
            k=None if k is None else c(k, dtype=np.float16).view(np.uint16),
            v=None if v is None else c(v, dtype=np.float16).view(np.uint16),
            cu_q=c(cu_q, dtype=np.int32), cu_k=c(cu_k, dtype=np.int32),
            cu_mtiles=c(cu_mtiles, dtype=np.int32), words=c(words, dtype=np.uint64),
            q8=c(q8, dtype=np.int8), q_scale=c(q_scale, dtype=np.float32),
            k8=c(k8, dtype=np.int8), k_scale=c(k_scale, dtype=np.float32),
            v8=None if v8 is None else c(v8, dtype=np.int8),
            v_scale=None if v_scale is None else c(v_scale, dtype=np.float32),
        )
        a = self.arrays
        self.hq, self.d = hq, d
        self.total_q = int(a["cu_q"][-1])
        self.total_mtiles = int(a["cu_mtiles"][-1])
        self.bm_r, self.bn_r = bm_r, bn_r
        self.problem = Problem(
            batch=len(a["cu_q"]) - 1, hq=hq, hk=hk, d=d,
            total_q=self.total_q, total_k=int(a["cu_k"][-1]),
            cu_q=_ptr(a["cu_q"]), cu_k=_ptr(a["cu_k"]), cu_mtiles=_ptr(a["cu_mtiles"]),
            total_mtiles=self.total_mtiles,
            q=_ptr(a["q"]), k=_ptr(a["k"]), v=_ptr(a["v"]),
            q8=_ptr(a["q8"]), q_scale=_ptr(a["q_scale"]),
            k8=_ptr(a["k8"]), k_scale=_ptr(a["k_scale"]),
            v8=_ptr(a["v8"]), v_scale=_ptr(a["v_scale"]),
            kv_int8=int(bool(kv_int8)), words=_ptr(a["words"]),
            wpr=int(a["words"].shape[-1]), bm_r=bm_r, bn_r=bn_r, group=group,
            causal=int(bool(causal)), softmax_scale=float(softmax_scale))

    def prefill(self, rows: Optional[np.ndarray] = None):
        """-> (out fp32 [n, hq, d], lse fp32 [hq, n], int8_pairs, legal_pairs)."""
        if rows is not None:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = self.total_q if rows is None else len(rows)
        out = np.empty((n, self.hq, self.d), dtype=np.float32)
        lse = np.empty((self.hq, n), dtype=np.float32)
        n8 = ctypes.c_int64(0)
        nall = ctypes.c_int64(0)
        rc = lib().oracle_prefill(ctypes.byref(self.problem), _ptr(rows), n, _ptr(out), _ptr(lse),
                                  ctypes.addressof(n8), ctypes.addressof(nall))
        if rc:
            raise ValueError("oracle_prefill rejected the problem")
        return out, lse, n8.value, nall.value

    def int32_tiles(self, head: int, m0: int, m_count: int, ntiles_max: int,
                    fill: int = np.iinfo(np.int32).min):
        dump = np.full((m_count, ntiles_max, self.bm_r, self.bn_r), fill, dtype=np.int32)
        rc = lib().oracle_int32_tiles(ctypes.byref(self.problem), head, m0, m_count, ntiles_max,
                                      _ptr(dump))
        if rc:
            raise ValueError("oracle_int32_tiles rejected its arguments")
        return dump


def prepare(w, *, k8=None, k_scale=None, v8=None, v_scale=None, words=None,
            softmax_scale: float = 0.0, q=None, k=None, v=None) -> Prepared:
    """Quantize Q (and K, or K and V for an INT8 cache) with the oracle's own quantizer, pack the
    route map with the oracle's own packer, and return a ready problem for workload ``w``."""
    q = w.q if q is None else q
    k = w.k if k is None else k
    v = w.v if v is None else v
    q8, qs = quantize_rows(q)
    if k8 is None:
        k8, k_scale = quantize_rows(k)
    if w.kv_int8 and v8 is None:
        v8, v_scale = quantize_rows(v)
    if words is None:
        words = pack_route(w.route, w.words_per_row)
    cu = w.cu_seqlens
    return Prepared(q=q, k=None if w.kv_int8 else k, v=None if w.kv_int8 else v,
                    cu_q=cu, cu_k=cu, cu_mtiles=w.cu_mtiles, hq=w.hq, hk=w.hk, d=w.d,
                    words=words, bm_r=w.bm_r, bn_r=w.bn_r, group=w.group, causal=w.causal,
                    q8=q8, q_scale=qs, k8=k8, k_scale=k_scale, v8=v8, v_scale=v_scale,
                    kv_int8=w.kv_int8, softmax_scale=softmax_scale)
