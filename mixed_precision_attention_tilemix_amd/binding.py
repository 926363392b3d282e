"""Thin ctypes binding of libtilemix.so (include/tilemix.h).

The functions here carry the C names and only marshal arguments: they take torch tensors that
already live on the GPU, pass their device pointers, sizes and the current HIP stream to the
library, and raise ``TilemixError`` on a non-OK status. Every step of the computation runs in
the library's HIP kernels; there is no fallback of any kind. If the library has not been built,
importing this module succeeds but the first call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtilemix.so")
_lib = None

TILEMIX_OK, TILEMIX_EINVAL, TILEMIX_EUNSUPPORTED, TILEMIX_ELAUNCH = 0, 1, 2, 3

# The entry points declared in include/tilemix.h.
EXPORTED = ("tilemix_last_error", "tilemix_version", "tilemix_quantize_qk",
            "tilemix_pack_route_mask", "tilemix_prefill_workspace_size", "tilemix_prefill_fwd",
            "tilemix_decode_workspace_size", "tilemix_decode_fwd", "tilemix_route_workspace_size",
            "tilemix_route_topk_maxabs", "tilemix_route_bernoulli", "tilemix_quantize_blocks",
            "tilemix_decode_fwd_noalloc", "tilemix_decode_noalloc_max_bytes", "tilemix_prefill_v_path")


class TilemixError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"tilemix status {status}: {message}")
        self.status = status


class FwdParams(ctypes.Structure):
    """Mirror of tilemix_fwd_params."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("batch", ctypes.c_int32),
        ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("total_q", ctypes.c_int64), ("total_k", ctypes.c_int64),
        ("max_seqlen_q", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
        ("cu_mtiles", ctypes.c_void_p),
        ("total_mtiles", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("q_stride_tok", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
        ("k", ctypes.c_void_p), ("k_stride_tok", ctypes.c_int64), ("k_stride_head", ctypes.c_int64),
        ("v", ctypes.c_void_p), ("v_stride_tok", ctypes.c_int64), ("v_stride_head", ctypes.c_int64),
        ("q8", ctypes.c_void_p), ("q_scale", ctypes.c_void_p),
        ("k8", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
        ("v8", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("kv_int8", ctypes.c_int32),
        ("route_words", ctypes.c_void_p),
        ("words_per_row", ctypes.c_int32),
        ("route_block_m", ctypes.c_int32), ("route_block_n", ctypes.c_int32),
        ("route_group", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("out", ctypes.c_void_p), ("out_dtype", ctypes.c_int32),
        ("lse", ctypes.c_void_p),
        ("debug_s32", ctypes.c_void_p),
        ("debug_head", ctypes.c_int32), ("debug_mtile_begin", ctypes.c_int32),
        ("debug_mtile_count", ctypes.c_int32), ("debug_ntiles_max", ctypes.c_int32),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
        ("k_scale_block", ctypes.c_int32),
        ("debug_sync_stages", ctypes.c_int32),
        ("state_fp16", ctypes.c_int32),
        ("v_path", ctypes.c_int32),
    ]


class RouteParams(ctypes.Structure):
    """Mirror of tilemix_route_params."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("batch", ctypes.c_int32), ("hkv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("max_seqlen_k", ctypes.c_int32),
        ("cu_seqlens_k", ctypes.c_void_p), ("cu_mtiles", ctypes.c_void_p),
        ("total_mtiles", ctypes.c_int32),
        ("route_block_n", ctypes.c_int32), ("route_group", ctypes.c_int32),
        ("fp16_per_mille", ctypes.c_int32),
        ("k", ctypes.c_void_p), ("k_stride_tok", ctypes.c_int64), ("k_stride_head", ctypes.c_int64),
        ("k8", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
        ("total_k", ctypes.c_int64), ("kv_int8", ctypes.c_int32),
        ("seed", ctypes.c_uint64),
        ("route_words", ctypes.c_void_p), ("words_per_row", ctypes.c_int32),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
    ]


def load(path: Optional[str] = None):
    """Load libtilemix.so (once). Raises FileNotFoundError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is missing: build it with python -m mixed_precision_attention_tilemix_amd.build "
                                "(hipcc, gfx950); there is no fallback path")
    L = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.tilemix_last_error.restype = ctypes.c_char_p
    L.tilemix_last_error.argtypes = []
    L.tilemix_version.restype = i32
    L.tilemix_version.argtypes = []
    L.tilemix_quantize_qk.restype = ctypes.c_int
    L.tilemix_quantize_qk.argtypes = [vp, i64, i32, i64, i64, vp, vp,
                                      vp, i64, i32, i64, i64, vp, vp, i32, vp]
    L.tilemix_quantize_blocks.restype = ctypes.c_int
    L.tilemix_quantize_blocks.argtypes = [vp, i64, i32, i64, i64, vp, i32, i32, i32, vp, vp, i32, vp]
    L.tilemix_pack_route_mask.restype = ctypes.c_int
    L.tilemix_pack_route_mask.argtypes = [vp, i64, i32, vp, i32, vp]
    L.tilemix_prefill_workspace_size.restype = ctypes.c_int
    L.tilemix_prefill_workspace_size.argtypes = [ctypes.POINTER(FwdParams), ctypes.POINTER(ctypes.c_int64)]
    L.tilemix_prefill_fwd.restype = ctypes.c_int
    L.tilemix_prefill_fwd.argtypes = [ctypes.POINTER(FwdParams), vp]
    L.tilemix_decode_workspace_size.restype = ctypes.c_int
    L.tilemix_decode_workspace_size.argtypes = [ctypes.POINTER(FwdParams), ctypes.POINTER(ctypes.c_int64)]
    L.tilemix_decode_fwd.restype = ctypes.c_int
    L.tilemix_decode_fwd.argtypes = [ctypes.POINTER(FwdParams), vp]
    L.tilemix_decode_fwd_noalloc.restype = ctypes.c_int
    L.tilemix_decode_fwd_noalloc.argtypes = [ctypes.POINTER(FwdParams), vp]
    L.tilemix_decode_noalloc_max_bytes.restype = i64
    L.tilemix_decode_noalloc_max_bytes.argtypes = []
    L.tilemix_prefill_v_path.restype = ctypes.c_int32
    L.tilemix_prefill_v_path.argtypes = [ctypes.POINTER(FwdParams)]
    for name in ("tilemix_route_topk_maxabs", "tilemix_route_bernoulli"):
        getattr(L, name).restype = ctypes.c_int
        getattr(L, name).argtypes = [ctypes.POINTER(RouteParams), vp]
    L.tilemix_route_workspace_size.restype = ctypes.c_int
    L.tilemix_route_workspace_size.argtypes = [ctypes.POINTER(RouteParams), ctypes.POINTER(ctypes.c_int64)]
    _lib = L
    return L


def _check(status: int):
    if status != TILEMIX_OK:
        raise TilemixError(status, load().tilemix_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tilemix takes device tensors only")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _tok_head_strides(x: torch.Tensor):
    if x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("expected [tokens, heads, head_dim] with unit channel stride")
    return x.stride(0), x.stride(1)


def last_error() -> str:
    return load().tilemix_last_error().decode()


def version() -> int:
    return int(load().tilemix_version())


def tilemix_quantize_qk(q: Optional[torch.Tensor] = None, q8: Optional[torch.Tensor] = None,
                        q_scale: Optional[torch.Tensor] = None, k: Optional[torch.Tensor] = None,
                        k8: Optional[torch.Tensor] = None, k_scale: Optional[torch.Tensor] = None,
                        stream=None) -> None:
    """q fp16 [T, Hq, d] -> q8 int8 [T, Hq, d], q_scale fp32 [Hq, T]; same for k (either optional)."""
    ref = q if q is not None else k
    d = ref.shape[2]
    qs = _tok_head_strides(q) if q is not None else (0, 0)
    ks = _tok_head_strides(k) if k is not None else (0, 0)
    _check(load().tilemix_quantize_qk(
        _ptr(q), q.shape[0] if q is not None else 0, q.shape[1] if q is not None else 0,
        qs[0], qs[1], _ptr(q8), _ptr(q_scale),
        _ptr(k), k.shape[0] if k is not None else 0, k.shape[1] if k is not None else 0,
        ks[0], ks[1], _ptr(k8), _ptr(k_scale), d, _stream(stream)))


def tilemix_quantize_blocks(x: torch.Tensor, x8: torch.Tensor, scale: torch.Tensor,
                            cu_seqlens: torch.Tensor, max_seqlen: int, block_rows: int,
                            stream=None) -> None:
    """x fp16 [T, H, d] -> x8 int8 [T, H, d], scale fp32 [H, T] with one scale per block of
    block_rows tokens of a sequence (repeated on each row)."""
    st = _tok_head_strides(x)
    _check(load().tilemix_quantize_blocks(_ptr(x), x.shape[0], x.shape[1], st[0], st[1],
                                          _ptr(cu_seqlens), cu_seqlens.shape[0] - 1, int(max_seqlen),
                                          int(block_rows), _ptr(x8), _ptr(scale), x.shape[2],
                                          _stream(stream)))


def tilemix_pack_route_mask(route: torch.Tensor, words: torch.Tensor, stream=None) -> None:
    """route uint8 [..., t_mask] -> words (int64 storage of uint64) [..., words_per_row]."""
    t_mask = route.shape[-1]
    rows = route.numel() // t_mask if t_mask else words.numel() // words.shape[-1]
    _check(load().tilemix_pack_route_mask(_ptr(route), rows, t_mask, _ptr(words),
                                          words.shape[-1], _stream(stream)))


def tilemix_prefill_workspace_size(*, batch: int, hkv: int, head_dim: int, total_k: int,
                                   kv_int8: bool) -> int:
    """Bytes of device workspace tilemix_prefill_fwd needs."""
    p = FwdParams()
    p.struct_size = ctypes.sizeof(FwdParams)
    p.batch, p.hkv, p.head_dim, p.total_k, p.kv_int8 = batch, hkv, head_dim, total_k, int(kv_int8)
    out = ctypes.c_int64(0)
    _check(load().tilemix_prefill_workspace_size(ctypes.byref(p), ctypes.byref(out)))
    return out.value


def _fwd_params(*, q, q8, q_scale, k8, k_scale, route_words, cu_seqlens_q, cu_seqlens_k,
                cu_mtiles, max_seqlen_q, max_seqlen_k, route_block_m, route_block_n, route_group,
                out, workspace, k, v, v8, v_scale, causal, softmax_scale, lse, debug_s32,
                debug_head, debug_mtile_begin, debug_mtile_count, k_scale_block=0,
                debug_sync_stages=False, state_fp16=False, v_path=0) -> FwdParams:
    kv_int8 = v8 is not None
    qs = _tok_head_strides(q)
    ks = _tok_head_strides(k) if k is not None else (0, 0)
    vs = _tok_head_strides(v) if v is not None else (0, 0)
    p = FwdParams()
    p.struct_size = ctypes.sizeof(FwdParams)
    p.batch = cu_seqlens_q.shape[0] - 1
    p.hq = q.shape[1]
    p.hkv = k8.shape[1]
    p.head_dim = q.shape[2]
    p.total_q = q.shape[0]
    p.total_k = k8.shape[0]
    p.max_seqlen_q = int(max_seqlen_q)
    p.max_seqlen_k = int(max_seqlen_k)
    p.cu_seqlens_q = _ptr(cu_seqlens_q)
    p.cu_seqlens_k = _ptr(cu_seqlens_k)
    p.cu_mtiles = _ptr(cu_mtiles)
    p.total_mtiles = route_words.shape[1]
    p.q, (p.q_stride_tok, p.q_stride_head) = _ptr(q), qs
    p.k, (p.k_stride_tok, p.k_stride_head) = _ptr(k), ks
    p.v, (p.v_stride_tok, p.v_stride_head) = _ptr(v), vs
    p.q8, p.q_scale = _ptr(q8), _ptr(q_scale)
    p.k8, p.k_scale = _ptr(k8), _ptr(k_scale)
    p.v8, p.v_scale = _ptr(v8), _ptr(v_scale)
    p.kv_int8 = int(kv_int8)
    p.route_words = _ptr(route_words)
    p.words_per_row = route_words.shape[2]
    p.route_block_m, p.route_block_n, p.route_group = route_block_m, route_block_n, route_group
    p.causal = int(bool(causal))
    p.softmax_scale = float(softmax_scale)
    p.out = _ptr(out)
    p.out_dtype = 1 if out.dtype == torch.float32 else 0
    p.lse = _ptr(lse)
    p.debug_s32 = _ptr(debug_s32)
    p.k_scale_block = int(k_scale_block)
    p.debug_sync_stages = int(bool(debug_sync_stages))
    p.state_fp16 = int(bool(state_fp16))
    p.v_path = int(v_path)
    if debug_s32 is not None:
        p.debug_head, p.debug_mtile_begin = debug_head, debug_mtile_begin
        p.debug_mtile_count, p.debug_ntiles_max = debug_mtile_count, debug_s32.shape[1]
    p.workspace = _ptr(workspace)
    p.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return p


def tilemix_prefill_fwd(*, q, q8, q_scale, k8, k_scale, route_words, cu_seqlens_q, cu_seqlens_k,
                        cu_mtiles, max_seqlen_q: int, max_seqlen_k: int, route_block_m: int,
                        route_block_n: int, route_group: int, out, workspace, k=None, v=None, v8=None,
                        v_scale=None, causal: bool = True, softmax_scale: float = 0.0, lse=None,
                        debug_s32=None, debug_head: int = 0, debug_mtile_begin: int = 0,
                        debug_mtile_count: int = 0, k_scale_block: int = 0,
                        debug_sync_stages: bool = False, state_fp16: bool = False, v_path: int = 0,
                        stream=None) -> None:
    """Fill tilemix_fwd_params from device tensors and call tilemix_prefill_fwd."""
    p = _fwd_params(q=q, q8=q8, q_scale=q_scale, k8=k8, k_scale=k_scale, route_words=route_words,
                    cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k, cu_mtiles=cu_mtiles,
                    max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k,
                    route_block_m=route_block_m, route_block_n=route_block_n,
                    route_group=route_group, out=out, workspace=workspace, k=k, v=v, v8=v8,
                    v_scale=v_scale, causal=causal, softmax_scale=softmax_scale, lse=lse,
                    debug_s32=debug_s32, debug_head=debug_head,
                    debug_mtile_begin=debug_mtile_begin, debug_mtile_count=debug_mtile_count,
                    k_scale_block=k_scale_block, debug_sync_stages=debug_sync_stages,
                    state_fp16=state_fp16, v_path=v_path)
    _check(load().tilemix_prefill_fwd(ctypes.byref(p), _stream(stream)))


def tilemix_decode_workspace_size(*, batch: int, hq: int, hkv: int, head_dim: int,
                                  max_seqlen_q: int, max_seqlen_k: int) -> int:
    """Bytes of device workspace tilemix_decode_fwd needs."""
    p = FwdParams()
    p.struct_size = ctypes.sizeof(FwdParams)
    p.batch, p.hq, p.hkv, p.head_dim = batch, hq, hkv, head_dim
    p.max_seqlen_q, p.max_seqlen_k = max_seqlen_q, max_seqlen_k
    out = ctypes.c_int64(0)
    _check(load().tilemix_decode_workspace_size(ctypes.byref(p), ctypes.byref(out)))
    return out.value


def tilemix_decode_fwd(*, q, q8, q_scale, k8, k_scale, v8, v_scale, route_words, cu_seqlens_q,
                       cu_seqlens_k, cu_mtiles, max_seqlen_q: int, max_seqlen_k: int,
                       route_block_m: int, route_block_n: int, route_group: int, out, workspace,
                       causal: bool = True, softmax_scale: float = 0.0, lse=None,
                       stream=None) -> None:
    """Fill tilemix_fwd_params (INT8 K/V cache) from device tensors and call tilemix_decode_fwd."""
    p = _fwd_params(q=q, q8=q8, q_scale=q_scale, k8=k8, k_scale=k_scale, route_words=route_words,
                    cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k, cu_mtiles=cu_mtiles,
                    max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k,
                    route_block_m=route_block_m, route_block_n=route_block_n,
                    route_group=route_group, out=out, workspace=workspace, k=None, v=None, v8=v8,
                    v_scale=v_scale, causal=causal, softmax_scale=softmax_scale, lse=lse,
                    debug_s32=None, debug_head=0, debug_mtile_begin=0, debug_mtile_count=0)
    _check(load().tilemix_decode_fwd(ctypes.byref(p), _stream(stream)))


def tilemix_decode_fwd_noalloc(*, q, q8, q_scale, k8, k_scale, v8, v_scale, route_words,
                               cu_seqlens_q, cu_seqlens_k, cu_mtiles, max_seqlen_q: int,
                               max_seqlen_k: int, route_block_m: int, route_block_n: int,
                               route_group: int, out, causal: bool = True,
                               softmax_scale: float = 0.0, lse=None, stream=None) -> None:
    """tilemix_decode_fwd_noalloc: the decode call on the library's own per-device scratch (no
    workspace argument)."""
    p = _fwd_params(q=q, q8=q8, q_scale=q_scale, k8=k8, k_scale=k_scale, route_words=route_words,
                    cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k, cu_mtiles=cu_mtiles,
                    max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k,
                    route_block_m=route_block_m, route_block_n=route_block_n,
                    route_group=route_group, out=out, workspace=None, k=None, v=None, v8=v8,
                    v_scale=v_scale, causal=causal, softmax_scale=softmax_scale, lse=lse,
                    debug_s32=None, debug_head=0, debug_mtile_begin=0, debug_mtile_count=0)
    _check(load().tilemix_decode_fwd_noalloc(ctypes.byref(p), _stream(stream)))


def tilemix_prefill_v_path(*, total_q: int, total_k: int, max_seqlen_k: int, hq: int, hkv: int,
                           causal: bool = True, v_path: int = 0) -> int:
    """The V path tilemix_prefill_fwd takes for these sizes: 1 (V^T pre-pass) or 2 (direct)."""
    p = FwdParams()
    p.struct_size = ctypes.sizeof(FwdParams)
    p.total_q, p.total_k, p.max_seqlen_k = total_q, total_k, max_seqlen_k
    p.hq, p.hkv, p.causal, p.v_path = hq, hkv, int(bool(causal)), v_path
    return int(load().tilemix_prefill_v_path(ctypes.byref(p)))


def tilemix_decode_noalloc_max_bytes() -> int:
    """Bytes of the per-device scratch of tilemix_decode_fwd_noalloc."""
    return int(load().tilemix_decode_noalloc_max_bytes())


def tilemix_route_workspace_size(*, batch: int, hkv: int, max_seqlen_k: int, route_block_n: int,
                                 route_group: int) -> int:
    """Bytes of device workspace tilemix_route_topk_maxabs needs."""
    p = RouteParams()
    p.struct_size = ctypes.sizeof(RouteParams)
    p.batch, p.hkv, p.max_seqlen_k = batch, hkv, max_seqlen_k
    p.route_block_n, p.route_group = route_block_n, route_group
    out = ctypes.c_int64(0)
    _check(load().tilemix_route_workspace_size(ctypes.byref(p), ctypes.byref(out)))
    return out.value


def _route_params(*, cu_seqlens_k, cu_mtiles, max_seqlen_k, route_block_n, route_group,
                  fp16_per_mille, route_words, hkv, head_dim=0, k=None, k8=None, k_scale=None,
                  seed=0, workspace=None) -> RouteParams:
    p = RouteParams()
    p.struct_size = ctypes.sizeof(RouteParams)
    p.batch = cu_seqlens_k.shape[0] - 1
    p.hkv = hkv
    p.head_dim = head_dim
    p.max_seqlen_k = int(max_seqlen_k)
    p.cu_seqlens_k, p.cu_mtiles = _ptr(cu_seqlens_k), _ptr(cu_mtiles)
    p.total_mtiles = route_words.shape[1]
    p.route_block_n, p.route_group = route_block_n, route_group
    p.fp16_per_mille = int(fp16_per_mille)
    if k is not None:
        p.k, (p.k_stride_tok, p.k_stride_head) = _ptr(k), _tok_head_strides(k)
        p.total_k = k.shape[0]
    if k8 is not None:
        p.k8, p.k_scale, p.kv_int8 = _ptr(k8), _ptr(k_scale), 1
        p.total_k = k8.shape[0]
    p.seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    p.route_words, p.words_per_row = _ptr(route_words), route_words.shape[2]
    p.workspace = _ptr(workspace)
    p.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return p


def tilemix_route_topk_maxabs(*, cu_seqlens_k, cu_mtiles, max_seqlen_k: int, route_block_n: int,
                              route_group: int, fp16_per_mille: int, route_words, workspace,
                              k=None, k8=None, k_scale=None, stream=None) -> None:
    """Top-k max|K| routing written as route words [hkv, total_mtiles, words_per_row].

    k: fp16 [T, hkv, d] (strided); or k8 int8 [T, hkv, d] with k_scale fp32 [hkv, T]."""
    ref = k if k is not None else k8
    p = _route_params(cu_seqlens_k=cu_seqlens_k, cu_mtiles=cu_mtiles, max_seqlen_k=max_seqlen_k,
                      route_block_n=route_block_n, route_group=route_group,
                      fp16_per_mille=fp16_per_mille, route_words=route_words, hkv=ref.shape[1],
                      head_dim=ref.shape[2], k=k, k8=k8, k_scale=k_scale, workspace=workspace)
    _check(load().tilemix_route_topk_maxabs(ctypes.byref(p), _stream(stream)))


def tilemix_route_bernoulli(*, cu_seqlens_k, cu_mtiles, max_seqlen_k: int, route_block_n: int,
                            route_group: int, fp16_per_mille: int, seed: int, route_words,
                            stream=None) -> None:
    """Coverage-budget Bernoulli routing (Philox4x32-10) written as route words."""
    p = _route_params(cu_seqlens_k=cu_seqlens_k, cu_mtiles=cu_mtiles, max_seqlen_k=max_seqlen_k,
                      route_block_n=route_block_n, route_group=route_group,
                      fp16_per_mille=fp16_per_mille, route_words=route_words,
                      hkv=route_words.shape[0], seed=seed)
    _check(load().tilemix_route_bernoulli(ctypes.byref(p), _stream(stream)))
