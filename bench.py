"""Benchmark of the routed prefill attention hot path on one MI355X.

One step = one pass of the whole hot path on the 32k-token causal GQA workload (32 query /
8 KV heads, head_dim 128, route tiles 128x128, 4 key tiles per routing bit, the 10% of key
groups with the largest max|K| on the FP16 path, K with 4 outlier channels x20):
tilemix_quantize_qk (Q and K) + tilemix_pack_route_mask + tilemix_prefill_fwd, with all
inputs resident in device memory. TFLOP/s counts 4 * head_dim * Hq flops per legal causal
(query, key) pair (QK^T and P.V, two flops per multiply-add), divided by the step time.

The JSON line also carries the roofline of the fused kernel (its own launch time from HIP
events on its stream, against the mixed FP16/INT8 MFMA peak) and the CPU oracle timed on a
bounded sample of query rows of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP16 = 2516.6   # TFLOP/s, dense FP16 MFMA, MI355X (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_INT8 = 5033.2   # TOP/s, dense INT8 MFMA
PEAK_HBM = 8000.0    # GB/s

WORKLOAD = "gqa32k"
CAL_BYTES = 256 << 20   # plain device copy of known size: calibrates the HBM byte counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_fwd_gqa32k_traffic.md")
KERNEL_SRC = os.path.join(ROOT, "mixed_precision_attention_tilemix_amd", "csrc", "prefill_fwd.hip")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_fwd_decode128k.md")
DECODE_SRC = os.path.join(ROOT, "mixed_precision_attention_tilemix_amd", "csrc", "decode.hip")
ROUTE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "route_topk_gqa32k.md")
ROUTE_SRC = os.path.join(ROOT, "mixed_precision_attention_tilemix_amd", "csrc", "route.hip")
QUANT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "quantize_gqa32k.md")
QUANT_SRC = os.path.join(ROOT, "mixed_precision_attention_tilemix_amd", "csrc", "quantize.hip")


# The pages' own prefill figures (TileMix page, Section 5.3 end-to-end throughput): whole-model
# prefill on another machine, quoted beside the kernel figures as context only; they are not the
# same metric and are not a target.
PAGES_CONTEXT = {
    "source": "TileMix page, Section 5.3: LLaMA 3.2 3B-Instruct prefill, 4k tokens, batch 8, "
              "end-to-end through the model (quantization, scale restoration and routing included)",
    "hardware": "NVIDIA A100 40GB",
    "unit": "K tokens/s",
    "flashattention_fp16": 14.33,
    "tilemix_75pct_groups_int8": 31.80,
    "tilemix_all_groups_int8": 29.80,
    "note": "whole-model throughput on other hardware; not comparable with kernel TFLOP/s",
}


def prefill_metric(w):
    """The metric string of a prefill workload, built from its shape (the 32k GQA workload gives
    the headline metric)."""
    def tokens(n):
        return f"{n // 1024}k" if n % 1024 == 0 else str(n)
    if w.batch == 1:
        where = f"L={tokens(w.seqlens[0])}"
    else:
        where = f"a varlen batch of {w.batch} sequences ({tokens(w.total) if w.total % 1024 == 0 else w.total} tokens)"
    kind = "MHA" if w.hq == w.hk else "GQA"
    extra = ", INT8 K/V cache" if w.kv_int8 else ""
    causal = "causal" if w.causal else "non-causal"
    return f"{causal} prefill attention TFLOPS & % MFMA roofline at {where}, d={w.d}, {kind}{extra}"


def measure_mfma_peaks(stream, blocks=4096, iters=2048, reps=5):
    """Dense MFMA rates this GPU reaches on the two shapes the fused kernel issues
    (libtilemix_peak.so: long runs of independent 32x32 MFMAs, nothing else in the loop). Returns
    {"int8": TOP/s, "fp16": TFLOP/s}, the best of `reps` timed launches each."""
    import ctypes
    import torch
    from mixed_precision_attention_tilemix_amd import build as pkg_build
    if not os.path.exists(pkg_build.PEAK_LIB):
        raise FileNotFoundError(f"{pkg_build.PEAK_LIB} is missing: build it with "
                                "python -m mixed_precision_attention_tilemix_amd.build")
    lib = ctypes.CDLL(pkg_build.PEAK_LIB)
    lib.tilemix_peak_mfma.restype = ctypes.c_int
    lib.tilemix_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    chains = lib.tilemix_peak_chains()
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    res = {}
    for kind, name, flops_per in ((0, "int8", 2 * 32 * 32 * 32), (1, "fp16", 2 * 32 * 32 * 16)):
        def launch():
            st = lib.tilemix_peak_mfma(kind, blocks, iters, ctypes.c_void_p(out.data_ptr()),
                                       ctypes.c_void_p(stream.cuda_stream))
            if st != 0:
                raise RuntimeError(f"tilemix_peak_mfma failed: {st}")
        launch()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        total = blocks * 4 * iters * chains * flops_per
        res[name] = round(total / (best * 1e-3) / 1e12, 1)
    return res


def summarize_trace(path, warmup, steps):
    """Per-kernel statistics of a rocprofv3 kernel trace (CSV) of one bench.py run, with the
    warm-up dispatches (the first `warmup` of each step kernel) apart from the timed ones; prints
    a markdown table."""
    import csv
    rows = list(csv.DictReader(open(path)))
    by = {}
    for r in rows:
        name = r.get("Kernel_Name") or r.get("KernelName") or r.get("Name")
        t0 = int(r.get("Start_Timestamp") or r.get("BeginNs"))
        t1 = int(r.get("End_Timestamp") or r.get("EndNs"))
        by.setdefault(name, []).append((t0, (t1 - t0) / 1e3))
    print("| Kernel | dispatches | warm-up avg (us) | timed dispatches | timed avg (us) | timed median (us) | timed min (us) | timed max (us) |")
    print("|---|---|---|---|---|---|---|---|")
    for name, v in sorted(by.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        v.sort()
        d = [x for _, x in v]
        if len(d) >= warmup + steps:
            warm, timed = d[:warmup], d[warmup:warmup + steps]
        else:
            warm, timed = [], d
        short = name if len(name) < 90 else name[:87] + "..."
        wavg = f"{np.mean(warm):.1f}" if warm else "-"
        print(f"| `{short}` | {len(d)} | {wavg} | {len(timed)} | {np.mean(timed):.1f} | "
              f"{np.median(timed):.1f} | {np.min(timed):.1f} | {np.max(timed):.1f} |")


def calibration_copy():
    """One plain device-to-device copy of CAL_BYTES (read CAL_BYTES, write CAL_BYTES), so that a
    rocprofv3 --pmc run of this script sees what FETCH_SIZE / WRITE_SIZE report for known bytes."""
    import torch
    src = torch.full((CAL_BYTES,), 1, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def measured_traffic(traffic_file=TRAFFIC_FILE, kernel_src=KERNEL_SRC):
    """HBM bytes per launch from a committed counter summary, or None when the summary is
    missing or was taken on a different kernel source."""
    import hashlib
    if not os.path.exists(traffic_file):
        return None
    digest = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    fields = {}
    for line in open(traffic_file):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != digest:
        return None
    try:
        return float(fields["fetch_bytes_per_launch"]) + float(fields["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def int8_pair_counts(w):
    """Legal (query, key) pairs per head routed to INT8, summed over heads, from the route map."""
    rep = w.hq // w.hk
    n8 = 0
    cm = w.cu_mtiles
    for b, L in enumerate(w.seqlens):
        span = w.bn_r * w.group
        for m in range(cm[b + 1] - cm[b]):
            i0, i1 = m * w.bm_r, min(L, (m + 1) * w.bm_r)
            for gj in range(w.t_mask):
                j0 = gj * span
                if j0 >= L:
                    break
                j1 = min(L, j0 + span)
                # pairs (i, j) with i in [i0, i1), j in [j0, j1), j <= i
                if w.causal:
                    ii = np.arange(i0, i1)
                    cnt = int(np.clip(np.minimum(ii + 1, j1) - j0, 0, None).sum())
                else:
                    cnt = (i1 - i0) * (j1 - j0)
                bits = w.route[:, cm[b] + m, gj]
                n8 += cnt * int(bits.sum()) * rep
    return n8


SAMPLE_PAIRS = 1e9  # legal (row, head, key) triples of the oracle's sample: about 15 s of host time


def _sample_rows(w, local, lens, stride, k):
    """k query rows per route row, evenly spaced from its first to its last row (offsets
    round(i (BM_r - 1) / (k - 1))), for every stride-th route row and the last one."""
    tiles = list(range(0, w.total_mtiles, stride))
    if tiles[-1] != w.total_mtiles - 1:
        tiles.append(w.total_mtiles - 1)
    offs = sorted(set(int(round(i * (w.bm_r - 1) / (k - 1))) for i in range(k)))
    rows = np.array(sorted(set(m * w.bm_r + o for m in tiles for o in offs if m * w.bm_r + o < w.total)),
                    dtype=np.int64)
    keys = local[rows] + 1 if w.causal else lens[rows]
    return rows, int(keys.sum()) * w.hq


def baseline_rows(w):
    """Query rows (global token indices) of the oracle's sample and how they were chosen.
    Returns (rows, stride, k): k rows per route row, evenly spaced from its first to its last
    row, for every stride-th route row and the last one. Start from 4 rows at stride 1. When that
    sample holds at most SAMPLE_PAIRS legal pairs, k grows (6, 8, 12, 16, 24, ... up to BM_r,
    i.e. every row) while the sample stays within the budget; otherwise the stride doubles until
    it fits."""
    starts = np.repeat(np.asarray(w.cu_seqlens[:-1], dtype=np.int64), np.diff(w.cu_seqlens))
    local = np.arange(w.total, dtype=np.int64) - starts  # sequence-local index of every token
    lens = np.repeat(np.diff(w.cu_seqlens), np.diff(w.cu_seqlens))
    k = min(4, w.bm_r)
    rows, pairs = _sample_rows(w, local, lens, 1, k)
    if pairs <= SAMPLE_PAIRS:
        while k < w.bm_r:
            k_next = min(w.bm_r, k * 3 // 2 if k & (k - 1) == 0 else k * 4 // 3)  # 4, 6, 8, 12, 16, 24, ...
            r2, p2 = _sample_rows(w, local, lens, 1, k_next)
            if p2 > SAMPLE_PAIRS:
                break
            rows, k = r2, k_next
        return rows, 1, k
    stride = 2
    while True:
        rows, pairs = _sample_rows(w, local, lens, stride, k)
        n_tiles = len(range(0, w.total_mtiles, stride)) + 1
        if pairs <= SAMPLE_PAIRS or n_tiles <= 2:
            return rows, stride, k
        stride *= 2


def oracle_problem(w, scale_blocks=None):
    """The oracle's problem for workload w: per-token codes, or with scale_blocks = (bq, bk) the
    oracle's block-wise codes of Q and K (K of the INT8 cache included)."""
    import oracle
    if scale_blocks is None:
        return oracle.prepare(w)
    bq, bk = scale_blocks
    q8, qs = oracle.quantize_blocks(w.q, w.cu_seqlens, bq)
    k8, ks = oracle.quantize_blocks(w.k, w.cu_seqlens, bk)
    extra = {}
    if w.kv_int8:
        v8, vs = oracle.quantize_rows(w.v)
        extra = dict(v8=v8, v_scale=vs)
    return oracle.Prepared(q=w.q, k=None if w.kv_int8 else w.k, v=None if w.kv_int8 else w.v,
                           cu_q=w.cu_seqlens, cu_k=w.cu_seqlens, cu_mtiles=w.cu_mtiles, hq=w.hq,
                           hk=w.hk, d=w.d, words=oracle.pack_route(w.route, w.words_per_row),
                           bm_r=w.bm_r, bn_r=w.bn_r, group=w.group, causal=w.causal, q8=q8,
                           q_scale=qs, k8=k8, k_scale=ks, kv_int8=w.kv_int8, **extra)


def cpu_baseline(w, prob, rows, stride, per_tile, scale_blocks=None):
    import oracle
    prep = oracle_problem(w, scale_blocks)
    t0 = time.perf_counter()
    out, _, n8, nall = prep.prefill(rows)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.d * nall  # nall counts (row, head, key) legal triples
    import torch
    gpu = prob.out[torch.from_numpy(rows).cuda()].cpu().numpy()
    err = float(np.abs(gpu.astype(np.float64) - out).max())
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": f"{len(rows)} query rows x {w.hq} heads ({per_tile} rows per {w.bm_r}-row route tile, "
                  f"evenly spaced from its first to its last row, for route tiles m = 0, {stride}, "
                  f"{2 * stride}, ... and the last one; {nall} legal pairs), fp64 oracle, {dt:.1f} s",
        "seconds": dt,
        "parity_max_abs_err_on_sample": err,
    }


def decode_bytes(w):
    """Algorithmic HBM bytes of one tilemix_decode_fwd call: every cached key / value row a query
    can see, read once per KV head (int8 K and V rows + their two fp32 scales), the new tokens'
    fp16 and int8 query rows + scale, and the fp16 outputs + LSE."""
    kv = 0
    for lq, lk in zip(w.q_lens, w.k_lens):
        if lq:
            kv += lk * w.hk * (2 * w.d + 8)
    q = w.total_q * w.hq * (3 * w.d + 4)
    out = w.total_q * w.hq * (2 * w.d + 4)
    return kv + q + out


def run_decode(args):
    """One step = tilemix_quantize_qk on the new tokens + tilemix_decode_fwd against the cache."""
    import torch
    from mixed_precision_attention_tilemix_amd import binding, workloads
    from mixed_precision_attention_tilemix_amd.runner import DeviceDecode

    binding.load()
    w = workloads.make_decode(args.workload)
    prob = DeviceDecode(w, out_dtype=torch.float16, fused_q=args.fused_q)
    stream = torch.cuda.current_stream()
    nbytes = decode_bytes(w)
    for _ in range(args.warmup):
        prob.step()
    torch.cuda.synchronize()
    # the serving loop: the step captured once into a HIP graph and replayed
    graph = prob.capture()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    graph_step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record(stream)
        prob.quantize()
        e1.record(stream)
        prob.decode()
        e2.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms = float(np.mean([e1.elapsed_time(e2) for _, e1, e2 in ev]))
    q_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1, _ in ev]))
    eager_step_ms = wall * 1e3 / args.steps
    step_ms = graph_step_ms
    gbps = nbytes / (step_ms * 1e-3) / 1e9
    dec_gbps = nbytes / (dec_ms * 1e-3) / 1e9
    result = {
        "metric": "routed decode over the INT8 K/V cache: effective HBM bandwidth",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 K/V, fp32 softmax and P.V",
        "data": "synthetic",
        "config": dict(w.describe(), out_dtype="fp16", q_quantization="fused" if args.fused_q else "once"),
        "tokens_per_s": round(w.total_q / (step_ms * 1e-3), 1),
        "step_mode": "HIP graph replay of the step",
        "eager_ms_per_step": round(eager_step_ms, 4),
        "decode_ms": round(dec_ms, 4),
        "quantize_q_ms": round(q_ms, 4),
        "roofline": {
            "kernel": "decode_chunk_kernel<128> + decode_merge_kernel<128> (the tilemix_decode_fwd call)",
            "bound": "hbm",
            "achieved": round(dec_gbps, 1),
            "peak": PEAK_HBM,
            "unit": "GB/s",
            "frac": round(dec_gbps / PEAK_HBM, 4),
            "traffic": measured_traffic(DECODE_TRAFFIC_FILE, DECODE_SRC) if w.name == "decode128k" else None,
            "bytes_per_launch": nbytes,
        },
    }
    if not args.no_cpu_baseline:
        import oracle
        q8, qs = oracle.quantize_rows(w.q)
        k8, ks = oracle.quantize_rows(w.k)
        v8, vs = oracle.quantize_rows(w.v)
        prep = oracle.Prepared(q=w.q, k=None, v=None, cu_q=w.cu_q, cu_k=w.cu_k, cu_mtiles=w.cu_mtiles,
                               hq=w.hq, hk=w.hk, d=w.d, words=oracle.pack_route(w.route, w.words_per_row),
                               bm_r=w.bm_r, bn_r=w.bn_r, group=w.group, causal=w.causal, q8=q8,
                               q_scale=qs, k8=k8, k_scale=ks, v8=v8, v_scale=vs, kv_int8=True)
        t1 = time.perf_counter()
        ref, _, _, nall = prep.prefill()
        dt = time.perf_counter() - t1
        gpu = prob.out.float().cpu().numpy()
        result["cpu_baseline"] = {
            "value": round(nbytes / dt / 1e9, 3),
            "unit": "GB/s",
            "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"the whole step ({w.total_q} new tokens x {w.hq} heads, {nall} legal pairs), "
                      f"fp64 oracle, {dt:.2f} s",
            "seconds": dt,
            "parity_max_abs_err": float(np.abs(gpu.astype(np.float64) - ref).max()),
        }
    print(json.dumps(result), flush=True)


def run_quantize(args):
    """One step = the quantize-once pass over the 32k GQA workload's Q and K (tilemix_quantize_qk,
    per-token scales); the block-wise form (tilemix_quantize_blocks, one scale per 128-token block
    of Q and of K) is timed beside it."""
    import torch
    from mixed_precision_attention_tilemix_amd import binding, workloads

    binding.load()
    w = workloads.make("gqa32k")
    dev = torch.device("cuda")
    T, d = w.total, w.d
    q = torch.from_numpy(w.q).to(dev)
    k = torch.from_numpy(w.k).to(dev)
    cu = torch.from_numpy(w.cu_seqlens).to(dev)
    q8 = torch.empty((T, w.hq, d), dtype=torch.int8, device=dev)
    k8 = torch.empty((T, w.hk, d), dtype=torch.int8, device=dev)
    qs = torch.empty((w.hq, T), dtype=torch.float32, device=dev)
    ks = torch.empty((w.hk, T), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def per_token():
        binding.tilemix_quantize_qk(q=q, q8=q8, q_scale=qs, k=k, k8=k8, k_scale=ks)

    def blocks():
        binding.tilemix_quantize_blocks(q, q8, qs, cu, T, 128)
        binding.tilemix_quantize_blocks(k, k8, ks, cu, T, 128)

    nbytes = T * (w.hq + w.hk) * (3 * d + 4)  # fp16 read + int8 write + fp32 scale per row

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        t0 = time.perf_counter()
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps, float(np.mean([a.elapsed_time(b) for a, b in ev]))

    step_ms, call_ms = timed(per_token)
    got_q8, got_qs = q8.cpu().numpy(), qs.cpu().numpy()
    blk_step_ms, blk_call_ms = timed(blocks)
    result = {
        "metric": "quantize-once pass (per-token symmetric INT8 of Q and K): effective HBM bandwidth",
        "value": round(nbytes / (step_ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 in, int8 + fp32 scale out",
        "data": "synthetic",
        "config": {"workload": "quantize_gqa32k", "tokens": T, "hq": w.hq, "hkv": w.hk, "head_dim": d},
        "quantize_qk_ms": round(call_ms, 4),
        "quantize_blocks_128_ms": round(blk_call_ms, 4),
        "quantize_blocks_128_gbps": round(nbytes / (blk_call_ms * 1e-3) / 1e9, 1),
        "roofline": {
            "kernel": "quantize_rows_kernel<128> (Q and K launches of the tilemix_quantize_qk call)",
            "bound": "hbm",
            "achieved": round(nbytes / (call_ms * 1e-3) / 1e9, 1),
            "peak": PEAK_HBM,
            "unit": "GB/s",
            "frac": round(nbytes / (call_ms * 1e-3) / 1e9 / PEAK_HBM, 4),
            "traffic": measured_traffic(QUANT_TRAFFIC_FILE, QUANT_SRC),
            "bytes_per_launch": nbytes,
        },
    }
    if not args.no_cpu_baseline:
        import oracle
        t1 = time.perf_counter()
        rq8, rqs = oracle.quantize_rows(w.q)
        oracle.quantize_rows(w.k)
        dt = time.perf_counter() - t1
        result["cpu_baseline"] = {
            "value": round(nbytes / dt / 1e9, 3),
            "unit": "GB/s",
            "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"the whole step (Q and K of {T} tokens), {dt:.2f} s",
            "seconds": dt,
            "parity_q_codes_equal": bool(np.array_equal(got_q8, rq8) and np.array_equal(got_qs, rqs.T)),
        }
    print(json.dumps(result), flush=True)


ROUTE_WORKLOADS = {"route_gqa32k": ("gqa32k", 100)}


def run_route(args):
    """One step = tilemix_route_topk_maxabs on the 32k GQA workload's K (top 10 % max|K| groups
    FP16), i.e. the on-device version of the policy that builds that workload's route map."""
    import torch
    from mixed_precision_attention_tilemix_amd import binding, workloads

    binding.load()
    base, per_mille = ROUTE_WORKLOADS[args.workload]
    w = workloads.make(base)
    dev = torch.device("cuda")
    k = torch.from_numpy(w.k).to(dev)
    cu = torch.from_numpy(w.cu_seqlens).to(dev)
    cu_m = torch.from_numpy(w.cu_mtiles).to(dev)
    words = torch.empty((w.hk, w.total_mtiles, w.words_per_row), dtype=torch.int64, device=dev)
    L = max(w.seqlens)
    nws = binding.tilemix_route_workspace_size(batch=w.batch, hkv=w.hk, max_seqlen_k=L,
                                               route_block_n=w.bn_r, route_group=w.group)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def topk():
        binding.tilemix_route_topk_maxabs(cu_seqlens_k=cu, cu_mtiles=cu_m, max_seqlen_k=L,
                                          route_block_n=w.bn_r, route_group=w.group,
                                          fp16_per_mille=per_mille, route_words=words, workspace=ws, k=k)

    def bern():
        binding.tilemix_route_bernoulli(cu_seqlens_k=cu, cu_mtiles=cu_m, max_seqlen_k=L,
                                        route_block_n=w.bn_r, route_group=w.group,
                                        fp16_per_mille=per_mille, seed=1, route_words=words)

    tmax = -(-L // (w.bn_r * w.group))
    nbytes = (w.total * w.hk * w.d * 2 + words.numel() * 8 + 2 * 4 * w.batch * w.hk * tmax)
    for _ in range(args.warmup):
        topk()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        topk()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    got = words.cpu().numpy().view(np.uint64)
    for e0, e1 in ev:
        e0.record(stream)
        bern()
        e1.record(stream)
    torch.cuda.synchronize()
    bern_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    step_ms = wall * 1e3 / args.steps
    result = {
        "metric": "on-device top-k max|K| routing fused with packing: effective HBM bandwidth",
        "value": round(nbytes / (step_ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 keys, fp32 group maxima",
        "data": "synthetic",
        "config": dict(w.describe(), workload=args.workload, fp16_per_mille=per_mille),
        "route_topk_ms": round(call_ms, 4),
        "route_bernoulli_ms": round(bern_ms, 4),
        "matches_host_route_map": None,
        "roofline": {
            "kernel": "group_maxabs_kernel<128,false> + topk_pack_kernel (the tilemix_route_topk_maxabs call)",
            "bound": "hbm",
            "achieved": round(nbytes / (call_ms * 1e-3) / 1e9, 1),
            "peak": PEAK_HBM,
            "unit": "GB/s",
            "frac": round(nbytes / (call_ms * 1e-3) / 1e9 / PEAK_HBM, 4),
            "traffic": measured_traffic(ROUTE_TRAFFIC_FILE, ROUTE_SRC),
            "bytes_per_launch": nbytes,
        },
    }
    if not args.no_cpu_baseline:
        import oracle
        t1 = time.perf_counter()
        R = oracle.route_topk_maxabs(w.cu_seqlens, w.cu_mtiles, w.hk, w.d, w.bn_r, w.group, per_mille,
                                     k=w.k, t_mask=w.t_mask)
        dt = time.perf_counter() - t1
        want = oracle.pack_route(R, w.words_per_row)
        result["matches_host_route_map"] = bool(np.array_equal(want, oracle.pack_route(w.route, w.words_per_row)))
        result["cpu_baseline"] = {
            "value": round(nbytes / dt / 1e9, 3),
            "unit": "GB/s",
            "cores": 1,
            "kind": "oracle",
            "sample": f"the whole step (top-k policy over all {w.total} keys x {w.hk} KV heads), {dt:.2f} s",
            "seconds": dt,
            "parity_words_equal": bool(np.array_equal(got, want)),
        }
    print(json.dumps(result), flush=True)


def exact_attention_cpu(w):
    """Causal softmax attention of the fp16 inputs in fp64 with plain PyTorch CPU ops: the
    reference of the deviation sweep (independent of the routed kernel and of the oracle)."""
    import torch
    L, d = w.total, w.d
    q = torch.from_numpy(w.q.astype(np.float64))
    k = torch.from_numpy(w.k.astype(np.float64))
    v = torch.from_numpy(w.v.astype(np.float64))
    out = torch.empty((L, w.hq, d), dtype=torch.float64)
    grp = w.hq // w.hk
    mask = torch.ones((L, L), dtype=torch.bool).tril()
    for h in range(w.hq):
        s = (q[:, h] @ k[:, h // grp].T) / np.sqrt(d)
        s.masked_fill_(~mask, float("-inf"))
        out[:, h] = torch.softmax(s, dim=-1) @ v[:, h // grp]
    return out.numpy()


def run_numerics(args):
    """Mean absolute output deviation of the routed kernel from exact attention, by sequence length
    and INT8 tile-group coverage (the paper's Table 3 study) on randomized inputs."""
    import torch
    from mixed_precision_attention_tilemix_amd import binding, workloads
    from mixed_precision_attention_tilemix_amd.runner import DeviceProblem

    binding.load()
    table = {}
    t0 = time.perf_counter()
    for L in workloads.NUMERICS_LENGTHS:
        exact = None
        row = {}
        for cov in workloads.NUMERICS_COVERAGES:
            w = workloads.numerics_case(L, cov)
            if exact is None:
                exact = exact_attention_cpu(w)
            prob = DeviceProblem(w, out_dtype=torch.float32)
            prob.step()
            torch.cuda.synchronize()
            out = prob.out.cpu().numpy().astype(np.float64)
            # the same inputs and routes with the online-softmax state kept in binary16
            prob.attention(state_fp16=True)
            torch.cuda.synchronize()
            out_s16 = prob.out.cpu().numpy().astype(np.float64)
            n8 = int8_pair_counts(w)
            del prob
            # the same point with per-block scales: one per 64-token block of Q and of K
            prob = DeviceProblem(w, out_dtype=torch.float32, scale_blocks=(w.bm_r, w.bn_r))
            prob.step()
            torch.cuda.synchronize()
            out_b = prob.out.cpu().numpy().astype(np.float64)
            del prob
            row[f"{int(round(100 * cov))}%"] = {
                "mean_abs_dev": float(np.abs(out - exact).mean()),
                "max_abs_dev": float(np.abs(out - exact).max()),
                "mean_abs_dev_block_scales": float(np.abs(out_b - exact).mean()),
                "mean_abs_dev_fp16_state": float(np.abs(out_s16 - exact).mean()),
                "max_abs_dev_fp16_state": float(np.abs(out_s16 - exact).max()),
                "int8_pair_fraction": round(n8 / (w.legal_pairs() * w.hq), 4),
            }
        table[str(L)] = row
    last = table[str(workloads.NUMERICS_LENGTHS[-1])][f"{int(round(100 * workloads.NUMERICS_COVERAGES[-1]))}%"]
    result = {
        "metric": "mean |O - O_exact| of routed prefill by INT8 tile-group coverage (randomized inputs)",
        "value": last["mean_abs_dev"],
        "unit": "abs",
        "n_gpus": 1,
        "higher_is_better": False,
        "data": "synthetic",
        "dtype": "fp16+int8 (fp32 accumulate), fp32 output",
        "config": {"workload": "numerics", "hq": 24, "hkv": 8, "head_dim": 128, "causal": True,
                   "route_tile": [64, 64], "group": 1, "lengths": list(workloads.NUMERICS_LENGTHS),
                   "int8_coverages": list(workloads.NUMERICS_COVERAGES),
                   "reference": "exact causal attention of the fp16 inputs, fp64, PyTorch CPU",
                   "scales": "per token (mean_abs_dev) and per 64-token block (mean_abs_dev_block_scales)",
                   "state": "fp32 online-softmax state, and binary16 state rounded after every 64-key "
                            "tile (*_fp16_state, per-token scales)"},
        "table": table,
        "seconds": round(time.perf_counter() - t0, 1),
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize-trace", default=None, metavar="KERNEL_TRACE_CSV",
                    help="print per-kernel statistics of a rocprofv3 kernel trace of a bench.py run "
                         "(warm-up dispatches apart from timed ones, by --warmup / --steps) and exit")
    ap.add_argument("--quantize-once", action="store_true",
                    help="quantize Q in a separate pass before the attention call (default: the "
                         "attention kernel quantizes Q itself, with bit-identical codes)")
    ap.add_argument("--scale-blocks", default=None, metavar="BQ,BK",
                    help="prefill on block-wise scales: Q and K quantized with one scale per BQ query / "
                         "BK key tokens of a sequence (tilemix_quantize_blocks); a BK multiple of 64 "
                         "lets the attention kernel take one K scale per key tile")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.warmup, args.steps)
        return
    args.scale_blocks = tuple(int(x) for x in args.scale_blocks.split(",")) if args.scale_blocks else None
    # Q stays fused (per token) when its blocks are single tokens
    args.fused_q = not args.quantize_once and (args.scale_blocks is None or args.scale_blocks[0] == 1)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by KV head with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    from mixed_precision_attention_tilemix_amd import workloads as _wl
    if args.workload == "numerics":
        run_numerics(args)
        return
    if args.workload in ROUTE_WORKLOADS:
        run_route(args)
        return
    if args.workload == "quantize_gqa32k":
        run_quantize(args)
        return
    if args.workload in _wl.DECODE_WORKLOADS:
        run_decode(args)
        return

    import torch
    from mixed_precision_attention_tilemix_amd import binding, workloads
    from mixed_precision_attention_tilemix_amd.runner import DeviceProblem

    binding.load()
    calibration_copy()
    w = workloads.make(args.workload)
    prob = DeviceProblem(w, out_dtype=torch.float16, fused_q=args.fused_q, scale_blocks=args.scale_blocks)
    stream = torch.cuda.current_stream()

    pairs_per_head = w.legal_pairs()
    pairs = pairs_per_head * w.hq
    n8 = int8_pair_counts(w)
    r = n8 / pairs
    flops = 4.0 * w.d * pairs
    # mixed floor: INT8 QK^T at the INT8 peak, FP16 QK^T and all P.V at the FP16 peak
    def mixed_peak(p_int8, p_fp16):
        t_floor = (2 * w.d * n8) / (p_int8 * 1e12) + (2 * w.d * (pairs - n8) + 2 * w.d * pairs) / (p_fp16 * 1e12)
        return flops / t_floor / 1e12
    peak_mixed = mixed_peak(PEAK_INT8, PEAK_FP16)

    for _ in range(args.warmup):
        prob.step()
    torch.cuda.synchronize()

    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, eq, e1, e2 in ev:
        e0.record(stream)
        prob.quantize()
        eq.record(stream)
        prob.pack()
        e1.record(stream)
        prob.attention()
        e2.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd = np.array([e1.elapsed_time(e2) for _, _, e1, e2 in ev])
    steps_ev = np.array([e0.elapsed_time(e2) for e0, _, _, e2 in ev])
    quant = np.array([e0.elapsed_time(eq) for e0, eq, _, _ in ev])
    fwd_ms = float(np.mean(fwd))
    pre_ms = float(np.mean([e0.elapsed_time(e1) for e0, _, e1, _ in ev]))
    quant_ms = float(np.median(quant))
    step_ms = wall * 1e3 / args.steps
    peaks = measure_mfma_peaks(stream)

    tflops = flops / (step_ms * 1e-3) / 1e12
    fwd_tflops = flops / (fwd_ms * 1e-3) / 1e12
    # fp16 read + int8 write + fp32 scale of the rows the quantize pass covers
    q_bytes = w.total * ((0 if args.fused_q else w.hq) + (0 if w.kv_int8 else w.hk)) * (w.d * 3 + 4)

    result = {
        "metric": prefill_metric(w),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16+int8 (fp32 accumulate)",
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.batch, "seq_len": w.seqlens[0] if w.batch == 1 else w.total,
            "hq": w.hq, "hkv": w.hk, "head_dim": w.d, "causal": w.causal,
            "route_tile": [w.bm_r, w.bn_r], "group": w.group, "policy": w.policy,
            "int8_pair_fraction": round(r, 4), "out_dtype": "fp16",
            "q_quantization": ("fused" if args.fused_q else "once") if args.scale_blocks is None
                              else f"blocks of {args.scale_blocks[0]} (Q) / {args.scale_blocks[1]} (K) tokens",
            "k_scale_block": prob.k_scale_block,
        },
        "pct_mixed_roofline": round(100 * tflops / peak_mixed, 2),
        "pct_fp16_roofline": round(100 * tflops / PEAK_FP16, 2),
        "ms_per_step_events": {"mean": round(float(np.mean(steps_ev)), 4),
                               "median": round(float(np.median(steps_ev)), 4),
                               "min": round(float(np.min(steps_ev)), 4)},
        "fwd_ms": round(fwd_ms, 4),
        "fwd_ms_median": round(float(np.median(fwd)), 4),
        "fwd_ms_min": round(float(np.min(fwd)), 4),
        "quantize_pack_ms": round(pre_ms, 4),
        "quantize_ms_median": round(quant_ms, 4),
        "quantize_gbps": round(q_bytes / (quant_ms * 1e-3) / 1e9, 1) if q_bytes else None,
        "roofline": {
            # instance 0 is the production kernel (per-key K scales), 2 the block-scale one
            # (last template argument: persistent launch, taken on the V^T path)
            "kernel": f"prefill_fwd_kernel<{w.d}, {str(bool(w.kv_int8)).lower()}, "
                      f"{2 if prob.k_scale_block > 0 else 0}, {str(prob.v_path() == 2).lower()}, "
                      f"{str(prob.v_path() == 1).lower()}>"
                      + (" (+ vt_pack pre-pass in the timed call)" if prob.v_path() == 1 else
                         " (+ cache_widen pre-pass in the timed call)" if w.kv_int8 else "")
                      + f"; V path {prob.v_path()}",
            "bound": "mfma",
            "achieved": round(fwd_tflops, 2),
            "peak": round(peak_mixed, 1),
            "unit": "TFLOP/s",
            "frac": round(fwd_tflops / peak_mixed, 4),
            "peak_measured": round(mixed_peak(peaks["int8"], peaks["fp16"]), 1),
            "frac_measured": round(fwd_tflops / mixed_peak(peaks["int8"], peaks["fp16"]), 4),
            "mfma_peaks": {"int8_spec": PEAK_INT8, "int8_measured": peaks["int8"],
                           "fp16_spec": PEAK_FP16, "fp16_measured": peaks["fp16"],
                           "how": "libtilemix_peak.so: 16384 wavefronts issuing 4 independent "
                                  "32x32 MFMA chains, best of 5 launches"},
            # the committed counters were taken on this workload's default configuration only
            "traffic": measured_traffic() if (args.workload == WORKLOAD and args.fused_q
                                              and args.scale_blocks is None) else None,
            "flops_per_launch": flops,
            "peak_note": f"mixed MFMA peak for INT8 fraction {r:.4f}: INT8 QK^T at {PEAK_INT8}, "
                         f"FP16 QK^T and P.V at {PEAK_FP16} TFLOP/s",
        },
    }
    result["context"] = PAGES_CONTEXT
    if not args.no_cpu_baseline:
        rows, stride, per_tile = baseline_rows(w)
        result["cpu_baseline"] = cpu_baseline(w, prob, rows, stride, per_tile, args.scale_blocks)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
