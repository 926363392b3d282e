"""Device-side plumbing around the three library calls: upload a workload, allocate the
outputs with torch, and run one pass of the hot path (quantize-once, pack, fused attention)."""

from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import binding as B


class DeviceProblem:
    """A workload resident in device memory plus its outputs.

    ``step()`` is one pass of the hot path: tilemix_quantize_qk (Q, and K unless K/V arrive as
    an INT8 cache), the route words, and tilemix_prefill_fwd, all enqueued on the current
    stream. The route words come from tilemix_pack_route_mask of the workload's routing map, or,
    with ``route_policy``, from an on-device policy computed in the step:
    ``("topk_maxabs", fp16_per_mille)`` or ``("bernoulli", fp16_per_mille, seed)``.
    With ``fused_q`` the fused kernel quantizes Q itself (q8 / q_scale passed as NULL) and the
    quantize step covers K only. With ``scale_blocks=(bq, bk)`` Q and K are quantized block-wise
    (tilemix_quantize_blocks: one scale per bq query / bk key tokens of a sequence) instead of
    per token (blocks of one token use the per-token pass; with ``fused_q`` the Q blocks must be one
    token); with an INT8 cache the blocks apply to the cached K. When the K block is a multiple
    of 64 keys, tilemix_prefill_fwd is told so (k_scale_block) and takes one K scale per key tile,
    unless ``k_block_tiles`` is False. With ``kv_int8`` the INT8 K/V cache is produced once at
    construction by the library's own quantizer, and the fp16 K/V are dropped."""

    def __init__(self, w, device: str = "cuda", out_dtype=torch.float32, with_lse: bool = True,
                 softmax_scale: float = 0.0, route_policy: Optional[tuple] = None,
                 fused_q: bool = False, scale_blocks: Optional[tuple] = None,
                 k_block_tiles: bool = True):
        if fused_q and scale_blocks is not None and scale_blocks[0] != 1:
            raise ValueError("fused Q quantization is per token; Q blocks must be 1 token with fused_q")
        self.w = w
        self.route_policy = route_policy
        self.fused_q = fused_q
        self.scale_blocks = scale_blocks
        # block-wise K scales on 64-key multiples: the kernel takes one K scale per key tile
        self.k_scale_block = (scale_blocks[1] if scale_blocks is not None and k_block_tiles
                              and scale_blocks[1] % 64 == 0 else 0)
        dev = torch.device(device)
        T, hq, hk, d = w.total, w.hq, w.hk, w.d
        self.q = torch.from_numpy(w.q).to(dev)
        self.cu = torch.from_numpy(w.cu_seqlens).to(dev)
        self.cu_mtiles = torch.from_numpy(w.cu_mtiles).to(dev)
        self.route = torch.from_numpy(np.ascontiguousarray(w.route)).to(dev)
        self.q8 = torch.empty((T, hq, d), dtype=torch.int8, device=dev)
        self.q_scale = torch.empty((hq, T), dtype=torch.float32, device=dev)
        self.k8 = torch.empty((T, hk, d), dtype=torch.int8, device=dev)
        self.k_scale = torch.empty((hk, T), dtype=torch.float32, device=dev)
        self.words = torch.empty((hk, w.total_mtiles, w.words_per_row), dtype=torch.int64, device=dev)
        self.out = torch.empty((T, hq, d), dtype=out_dtype, device=dev)
        self.lse = torch.empty((hq, T), dtype=torch.float32, device=dev) if with_lse else None
        self.softmax_scale = softmax_scale
        self.max_seqlen = max(w.seqlens) if w.seqlens else 0
        ws_bytes = B.tilemix_prefill_workspace_size(batch=w.batch, hkv=hk, head_dim=d, total_k=T,
                                                    kv_int8=w.kv_int8)
        self.workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.route_ws = None
        if route_policy is not None and route_policy[0] == "topk_maxabs":
            n = B.tilemix_route_workspace_size(batch=w.batch, hkv=hk, max_seqlen_k=max(w.seqlens),
                                               route_block_n=w.bn_r, route_group=w.group)
            self.route_ws = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        if w.kv_int8:
            k = torch.from_numpy(w.k).to(dev)
            v = torch.from_numpy(w.v).to(dev)
            self.v8 = torch.empty((T, hk, d), dtype=torch.int8, device=dev)
            self.v_scale = torch.empty((hk, T), dtype=torch.float32, device=dev)
            B.tilemix_quantize_qk(q=v, q8=self.v8, q_scale=self.v_scale, k=k, k8=self.k8,
                                  k_scale=self.k_scale)
            if scale_blocks is not None:
                B.tilemix_quantize_blocks(k, self.k8, self.k_scale, self.cu, self.max_seqlen,
                                          scale_blocks[1])
            del k, v
            self.k = self.v = None
        else:
            self.k = torch.from_numpy(w.k).to(dev)
            self.v = torch.from_numpy(w.v).to(dev)
            self.v8 = self.v_scale = None

    def quantize(self, stream=None):
        if self.scale_blocks is not None:
            # blocks of one token are the per-token quantizer (same codes and scales): that pass,
            # or for Q with fused_q the fused kernel itself
            bq, bk = self.scale_blocks
            if not self.fused_q:
                if bq == 1:
                    B.tilemix_quantize_qk(q=self.q, q8=self.q8, q_scale=self.q_scale, stream=stream)
                else:
                    B.tilemix_quantize_blocks(self.q, self.q8, self.q_scale, self.cu, self.max_seqlen, bq,
                                              stream=stream)
            if not self.w.kv_int8:
                if bk == 1:
                    B.tilemix_quantize_qk(k=self.k, k8=self.k8, k_scale=self.k_scale, stream=stream)
                else:
                    B.tilemix_quantize_blocks(self.k, self.k8, self.k_scale, self.cu, self.max_seqlen, bk,
                                              stream=stream)
            return
        qargs = {} if self.fused_q else dict(q=self.q, q8=self.q8, q_scale=self.q_scale)
        if not self.w.kv_int8:
            qargs.update(k=self.k, k8=self.k8, k_scale=self.k_scale)
        if qargs:
            B.tilemix_quantize_qk(stream=stream, **qargs)

    def pack(self, stream=None):
        B.tilemix_pack_route_mask(self.route.view(-1, self.route.shape[-1]),
                                  self.words.view(-1, self.words.shape[-1]), stream=stream)

    def route_words(self, stream=None):
        """Fill the route words: pack the workload's map, or run the on-device policy."""
        pol = self.route_policy
        if pol is None:
            self.pack(stream)
            return
        w = self.w
        common = dict(cu_seqlens_k=self.cu, cu_mtiles=self.cu_mtiles, max_seqlen_k=self.max_seqlen,
                      route_block_n=w.bn_r, route_group=w.group, fp16_per_mille=pol[1],
                      route_words=self.words, stream=stream)
        if pol[0] == "topk_maxabs":
            if w.kv_int8:
                B.tilemix_route_topk_maxabs(k8=self.k8, k_scale=self.k_scale, workspace=self.route_ws, **common)
            else:
                B.tilemix_route_topk_maxabs(k=self.k, workspace=self.route_ws, **common)
        elif pol[0] == "bernoulli":
            B.tilemix_route_bernoulli(seed=pol[2], **common)
        else:
            raise ValueError(f"unknown route policy {pol[0]!r}")

    def attention(self, stream=None, debug_s32: Optional[torch.Tensor] = None, debug_head: int = 0,
                  debug_mtile_begin: int = 0, debug_mtile_count: int = 0,
                  debug_sync_stages: bool = False, state_fp16: bool = False, v_path: int = 0):
        w = self.w
        B.tilemix_prefill_fwd(
            q=self.q, k=self.k, v=self.v, q8=None if self.fused_q else self.q8,
            q_scale=None if self.fused_q else self.q_scale, k8=self.k8,
            k_scale=self.k_scale, v8=self.v8, v_scale=self.v_scale, route_words=self.words,
            cu_seqlens_q=self.cu, cu_seqlens_k=self.cu, cu_mtiles=self.cu_mtiles,
            max_seqlen_q=self.max_seqlen, max_seqlen_k=self.max_seqlen, route_block_m=w.bm_r,
            route_block_n=w.bn_r, route_group=w.group, causal=w.causal,
            softmax_scale=self.softmax_scale, out=self.out, lse=self.lse, workspace=self.workspace,
            debug_s32=debug_s32,
            debug_head=debug_head, debug_mtile_begin=debug_mtile_begin,
            debug_mtile_count=debug_mtile_count, k_scale_block=self.k_scale_block,
            debug_sync_stages=debug_sync_stages, state_fp16=state_fp16, v_path=v_path, stream=stream)

    def step(self, stream=None):
        self.quantize(stream)
        self.route_words(stream)
        self.attention(stream)

    def v_path(self) -> int:
        """The V path attention() takes by default: 1 (V^T pre-pass) or 2 (direct)."""
        w = self.w
        return B.tilemix_prefill_v_path(total_q=w.total, total_k=w.total, max_seqlen_k=self.max_seqlen,
                                        hq=w.hq, hkv=w.hk, causal=w.causal)


class DeviceDecode:
    """A decode workload in device memory: fp16 Q of the new tokens, the INT8 K/V cache
    (quantized once at construction by the library's own quantizer; the fp16 K/V are dropped),
    the packed route words and the outputs.

    ``step()`` is one decode step: tilemix_quantize_qk on the new query tokens, then
    tilemix_decode_fwd against the cache, both on the current stream. With ``fused_q`` the
    decode kernel quantizes the new tokens itself and the step is the decode call alone."""

    def __init__(self, w, device: str = "cuda", out_dtype=torch.float16, with_lse: bool = True,
                 fused_q: bool = False):
        dev = torch.device(device)
        self.w = w
        self.fused_q = fused_q
        hq, hk, d = w.hq, w.hk, w.d
        self.q = torch.from_numpy(w.q).to(dev)
        self.q8 = torch.empty((w.total_q, hq, d), dtype=torch.int8, device=dev)
        self.q_scale = torch.empty((hq, w.total_q), dtype=torch.float32, device=dev)
        self.k8 = torch.empty((w.total_k, hk, d), dtype=torch.int8, device=dev)
        self.k_scale = torch.empty((hk, w.total_k), dtype=torch.float32, device=dev)
        self.v8 = torch.empty((w.total_k, hk, d), dtype=torch.int8, device=dev)
        self.v_scale = torch.empty((hk, w.total_k), dtype=torch.float32, device=dev)
        if w.total_k:
            k = torch.from_numpy(w.k).to(dev)
            v = torch.from_numpy(w.v).to(dev)
            B.tilemix_quantize_qk(q=v, q8=self.v8, q_scale=self.v_scale, k=k, k8=self.k8,
                                  k_scale=self.k_scale)
            del k, v
        route = torch.from_numpy(np.ascontiguousarray(w.route)).to(dev)
        self.words = torch.empty((hk, route.shape[1], w.words_per_row), dtype=torch.int64, device=dev)
        B.tilemix_pack_route_mask(route, self.words)
        self.cu_q = torch.from_numpy(w.cu_q).to(dev)
        self.cu_k = torch.from_numpy(w.cu_k).to(dev)
        self.cu_mtiles = torch.from_numpy(w.cu_mtiles).to(dev)
        self.max_q = max(w.q_lens) if w.q_lens else 0
        self.max_k = max(w.k_lens) if w.k_lens else 0
        n = B.tilemix_decode_workspace_size(batch=w.batch, hq=hq, hkv=hk, head_dim=d,
                                            max_seqlen_q=self.max_q, max_seqlen_k=self.max_k)
        self.workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        self.out = torch.empty((w.total_q, hq, d), dtype=out_dtype, device=dev)
        self.lse = torch.empty((hq, w.total_q), dtype=torch.float32, device=dev) if with_lse else None

    def quantize(self, stream=None):
        if self.w.total_q and not self.fused_q:
            B.tilemix_quantize_qk(q=self.q, q8=self.q8, q_scale=self.q_scale, stream=stream)

    def decode(self, softmax_scale: float = 0.0, stream=None):
        w = self.w
        B.tilemix_decode_fwd(q=self.q, q8=None if self.fused_q else self.q8,
                             q_scale=None if self.fused_q else self.q_scale, k8=self.k8,
                             k_scale=self.k_scale, v8=self.v8, v_scale=self.v_scale,
                             route_words=self.words, cu_seqlens_q=self.cu_q, cu_seqlens_k=self.cu_k,
                             cu_mtiles=self.cu_mtiles, max_seqlen_q=self.max_q,
                             max_seqlen_k=self.max_k, route_block_m=w.bm_r, route_block_n=w.bn_r,
                             route_group=w.group, out=self.out, workspace=self.workspace,
                             causal=w.causal, softmax_scale=softmax_scale, lse=self.lse,
                             stream=stream)

    def step(self, stream=None):
        self.quantize(stream)
        self.decode(stream=stream)

    def capture(self):
        """Record one step into a HIP graph (torch.cuda.CUDAGraph) and return it; replaying it
        runs the step on the current contents of the input tensors (new query tokens written into
        ``self.q`` in place are picked up). The step's kernels clear nothing with memset, so the
        graph holds kernel nodes only."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm-up outside the capture, as the capture API asks
            self.step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.step()
        return graph
