"""Host-side logic of bench.py that runs without a GPU: the oracle's row sample, the legal-pair
counts behind the roofline, and the quoted context figures."""

from types import SimpleNamespace

import numpy as np
import pytest

import bench
from mixed_precision_attention_tilemix_amd import workloads as wl


def legal_keys(w, rows):
    """Legal keys of each sampled query row (sequence-local causal prefix, or the whole sequence)."""
    cu = np.asarray(w.cu_seqlens, dtype=np.int64)
    b = np.searchsorted(cu, rows, side="right") - 1
    local = rows - cu[b]
    return local + 1 if w.causal else (cu[b + 1] - cu[b])


@pytest.mark.parametrize("name", ["tiny", "mha8k", "gqa32k", "varlen64k"])
def test_baseline_rows_sample(name):
    w = wl.make(name)
    rows, stride, k = bench.baseline_rows(w)
    assert rows.dtype == np.int64 and rows.ndim == 1 and len(rows) > 0
    assert np.all(np.diff(rows) > 0), "rows sorted and unique"
    assert rows[0] == 0 and rows[-1] < w.total
    assert rows[-1] >= w.total - 2 * w.bm_r, "the sample reaches the end of the token range"
    pairs = int(legal_keys(w, rows).sum()) * w.hq
    assert pairs <= bench.SAMPLE_PAIRS
    assert stride >= 1 and stride & (stride - 1) == 0
    assert 4 <= k <= w.bm_r and (stride == 1 or k == 4)


def shape_only(seqlens, hq, bm_r=128, causal=True):
    """The fields baseline_rows reads, without generating tensors."""
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)
    mt = sum(-(-L // bm_r) for L in seqlens)
    return SimpleNamespace(cu_seqlens=cu, total=int(cu[-1]), total_mtiles=mt, bm_r=bm_r,
                           causal=causal, hq=hq)


def test_baseline_rows_stride_grows_with_size():
    _, s_small, k_small = bench.baseline_rows(shape_only([8192], 32))
    rows, s_big, k_big = bench.baseline_rows(shape_only([131072], 32))
    assert s_small == 1 and s_big > 1 and k_big == 4
    assert int(legal_keys(shape_only([131072], 32), rows).sum()) * 32 <= bench.SAMPLE_PAIRS


def test_baseline_rows_fill_the_budget():
    # a small workload is sampled in full; a mid-size one takes more rows per route tile, close to
    # the budget, before any stride is used
    w = shape_only([300, 77], 4, bm_r=64)
    rows, stride, k = bench.baseline_rows(w)
    assert stride == 1 and k == 64 and np.array_equal(rows, np.arange(377))
    w = shape_only([32768], 32)
    rows, stride, k = bench.baseline_rows(w)
    pairs = int(legal_keys(w, rows).sum()) * 32
    assert stride == 1 and k > 4 and 0.5 * bench.SAMPLE_PAIRS < pairs <= bench.SAMPLE_PAIRS
    offs = sorted(set(int(r) % 128 for r in rows))
    assert offs[0] == 0 and offs[-1] == 127 and len(offs) == k


def test_int8_pair_counts_closed_forms():
    # all-INT8 and all-FP16 routing: the INT8 count is every legal pair or none
    for route, frac in (("int8", 1.0), ("fp16", 0.0)):
        w = wl.custom([300, 77, 513], 4, 2, 64, bm_r=64, bn_r=64, route=route, seed=1)
        n8 = bench.int8_pair_counts(w)
        total = sum(L * (L + 1) // 2 for L in w.seqlens) * w.hq
        assert n8 == int(frac * total)


def test_pages_context_is_marked_as_context():
    c = bench.PAGES_CONTEXT
    assert c["hardware"].startswith("NVIDIA A100")
    assert c["flashattention_fp16"] == 14.33 and c["tilemix_75pct_groups_int8"] == 31.80
    assert "not comparable" in c["note"]


def test_prefill_metric_strings():
    """The headline workload carries the headline metric; the others name their own shape."""
    assert bench.prefill_metric(wl.make("gqa32k")) == \
        "causal prefill attention TFLOPS & % MFMA roofline at L=32k, d=128, GQA"
    assert bench.prefill_metric(wl.make("mha8k")).endswith("at L=8k, d=128, MHA")
    assert "INT8 K/V cache" in bench.prefill_metric(wl.make("kvint8_128k"))
    assert "varlen batch of 8 sequences" in bench.prefill_metric(wl.make("varlen64k"))
    assert bench.prefill_metric(wl.make("tiny")).endswith("at L=256, d=64, MHA")


def test_summarize_trace_splits_warmup(tmp_path, capsys):
    """Warm-up dispatches (the first `warmup` of each kernel) are reported apart from the timed ones."""
    path = tmp_path / "kernel_trace.csv"
    lines = ["Kernel_Name,Start_Timestamp,End_Timestamp"]
    t = 0
    for i in range(5):  # 2 warm-up + 3 timed dispatches of one kernel: 9 us, then 4 us each
        d = 9000 if i < 2 else 4000
        lines.append(f"k<1>,{t},{t + d}")
        t += 10000
    path.write_text("\n".join(lines) + "\n")
    bench.summarize_trace(str(path), warmup=2, steps=3)
    out = capsys.readouterr().out
    row = [r for r in out.splitlines() if r.startswith("| `k<1>`")][0]
    cells = [c.strip() for c in row.split("|")[1:-1]]
    assert cells[1] == "5" and cells[2] == "9.0" and cells[3] == "3" and cells[4] == "4.0"
