"""CPU-side checks of the C ABI: the library loads, exports every declared entry point, the
ctypes mirror of tilemix_fwd_params matches the C layout, and argument validation rejects bad
calls before any device work (no GPU is touched by these tests)."""

import ctypes
import os
import re
import subprocess

import pytest

from mixed_precision_attention_tilemix_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tilemix.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from mixed_precision_attention_tilemix_amd import build
        build.build()
    return B.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(tilemix_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("tilemix_quantize_qk", "tilemix_pack_route_mask", "tilemix_prefill_fwd",
              "tilemix_decode_fwd"):
        assert n in names
    assert set(names) == set(B.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True).stdout
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_params_struct_matches_c_layout(tmp_path):
    fields = [f for f, _ in B.FwdParams._fields_]
    src = tmp_path / "layout.c"
    body = "\n".join(f'  printf("%s %zu\\n", "{f}", offsetof(tilemix_fwd_params, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "tilemix.h"\nint main(void){\n'
                   '  printf("sizeof %zu\\n", sizeof(tilemix_fwd_params));\n' + body + "\n  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = dict(line.split() for line in subprocess.check_output([str(exe)], text=True).splitlines())
    assert int(got["sizeof"]) == ctypes.sizeof(B.FwdParams)
    for f in fields:
        assert int(got[f]) == getattr(B.FwdParams, f).offset, f


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def base_params():
    p = B.FwdParams()
    p.struct_size = ctypes.sizeof(B.FwdParams)
    p.batch, p.hq, p.hkv, p.head_dim = 1, 4, 2, 128
    p.total_q = p.total_k = 256
    p.max_seqlen_q = p.max_seqlen_k = 256
    p.cu_seqlens_q = p.cu_seqlens_k = p.cu_mtiles = FAKE
    p.total_mtiles = 2
    p.q = p.k = p.v = FAKE
    p.q_stride_tok, p.q_stride_head = 4 * 128, 128
    p.k_stride_tok, p.k_stride_head = 2 * 128, 128
    p.v_stride_tok, p.v_stride_head = 2 * 128, 128
    p.q8 = p.q_scale = p.k8 = p.k_scale = FAKE
    p.route_words = FAKE
    p.words_per_row = 1
    p.route_block_m, p.route_block_n, p.route_group = 128, 128, 1
    p.causal = 1
    p.out = FAKE
    p.workspace = FAKE
    p.workspace_bytes = 1 << 40
    return p


def int8_cache(p):
    """Switch base_params to an INT8 K/V cache (the only prefill mode with a workspace)."""
    p.kv_int8 = 1
    p.k = p.v = None
    p.v8 = p.v_scale = FAKE


BAD_CASES = [
    ("struct_size", lambda p: setattr(p, "struct_size", 8), B.TILEMIX_EINVAL),
    ("head_dim", lambda p: setattr(p, "head_dim", 96), B.TILEMIX_EUNSUPPORTED),
    ("gqa ratio", lambda p: setattr(p, "hkv", 3), B.TILEMIX_EINVAL),
    ("route_block_m", lambda p: setattr(p, "route_block_m", 48), B.TILEMIX_EINVAL),
    ("route_block_n", lambda p: setattr(p, "route_block_n", 96), B.TILEMIX_EINVAL),
    ("route_group", lambda p: setattr(p, "route_group", 0), B.TILEMIX_EINVAL),
    ("too many groups", lambda p: setattr(p, "max_seqlen_k", 128 * 65), B.TILEMIX_EINVAL),
    ("null q8 only", lambda p: setattr(p, "q8", None), B.TILEMIX_EINVAL),
    ("null q_scale only", lambda p: setattr(p, "q_scale", None), B.TILEMIX_EINVAL),
    ("null out", lambda p: setattr(p, "out", None), B.TILEMIX_EINVAL),
    ("kv_int8 with fp16 k", lambda p: setattr(p, "kv_int8", 1), B.TILEMIX_EINVAL),
    ("fp16 without v", lambda p: setattr(p, "v", None), B.TILEMIX_EINVAL),
    ("odd stride", lambda p: setattr(p, "q_stride_head", 4), B.TILEMIX_EINVAL),
    ("huge v token stride", lambda p: setattr(p, "v_stride_tok", 1 << 24), B.TILEMIX_EINVAL),
    ("misaligned q", lambda p: setattr(p, "q", FAKE + 2), B.TILEMIX_EINVAL),
    ("out dtype", lambda p: setattr(p, "out_dtype", 7), B.TILEMIX_EINVAL),
    ("null workspace", lambda p: (int8_cache(p), setattr(p, "workspace", None)), B.TILEMIX_EINVAL),
    ("small workspace", lambda p: (int8_cache(p), setattr(p, "workspace_bytes", 1024)), B.TILEMIX_EINVAL),
    ("misaligned workspace", lambda p: (int8_cache(p), setattr(p, "workspace", FAKE + 16)), B.TILEMIX_EINVAL),
    ("null workspace on the V^T path", lambda p: (setattr(p, "v_path", 1), setattr(p, "workspace", None)),
     B.TILEMIX_EINVAL),
    ("v_path", lambda p: setattr(p, "v_path", 3), B.TILEMIX_EINVAL),
    ("debug range", lambda p: (setattr(p, "debug_s32", FAKE), setattr(p, "debug_head", 9),
                               setattr(p, "debug_ntiles_max", 2)), B.TILEMIX_EINVAL),
    ("debug ntiles", lambda p: (setattr(p, "debug_s32", FAKE), setattr(p, "debug_mtile_count", 1),
                                setattr(p, "debug_ntiles_max", 1)), B.TILEMIX_EINVAL),
    ("sync with state_fp16", lambda p: (setattr(p, "debug_sync_stages", 1), setattr(p, "state_fp16", 1)),
     B.TILEMIX_EINVAL),
    ("dump with sync", lambda p: (setattr(p, "debug_s32", FAKE), setattr(p, "debug_mtile_count", 1),
                                  setattr(p, "debug_ntiles_max", 2), setattr(p, "debug_sync_stages", 1)),
     B.TILEMIX_EINVAL),
    ("dump with state_fp16", lambda p: (setattr(p, "debug_s32", FAKE), setattr(p, "debug_mtile_count", 1),
                                        setattr(p, "debug_ntiles_max", 2), setattr(p, "state_fp16", 1)),
     B.TILEMIX_EINVAL),
    ("k_scale_block negative", lambda p: setattr(p, "k_scale_block", -64), B.TILEMIX_EINVAL),
    ("k_scale_block not a tile multiple", lambda p: setattr(p, "k_scale_block", 96), B.TILEMIX_EINVAL),
]


@pytest.mark.parametrize("name,mutate,status", BAD_CASES, ids=[c[0] for c in BAD_CASES])
def test_prefill_validation(lib, name, mutate, status):
    p = base_params()
    mutate(p)
    got = lib.tilemix_prefill_fwd(ctypes.byref(p), None)
    assert got == status, (name, B.last_error())
    assert B.last_error()


def test_prefill_null_params(lib):
    assert lib.tilemix_prefill_fwd(None, None) == B.TILEMIX_EINVAL


def test_quantize_validation(lib):
    L = lib
    # unsupported head_dim
    assert L.tilemix_quantize_qk(FAKE, 8, 2, 256, 128, FAKE, FAKE, None, 0, 0, 0, 0, None, None,
                                 96, None) == B.TILEMIX_EUNSUPPORTED
    # input without outputs
    assert L.tilemix_quantize_qk(FAKE, 8, 2, 256, 128, None, FAKE, None, 0, 0, 0, 0, None, None,
                                 128, None) == B.TILEMIX_EINVAL
    # stride not a multiple of 8 elements
    assert L.tilemix_quantize_qk(FAKE, 8, 2, 256, 129, FAKE, FAKE, None, 0, 0, 0, 0, None, None,
                                 128, None) == B.TILEMIX_EINVAL
    # misaligned input
    assert L.tilemix_quantize_qk(None, 0, 0, 0, 0, None, None, FAKE + 8, 8, 2, 256, 128, FAKE,
                                 FAKE, 128, None) == B.TILEMIX_EINVAL
    assert "misaligned" in B.last_error()


def test_pack_validation(lib):
    assert lib.tilemix_pack_route_mask(FAKE, 4, 65, FAKE, 1, None) == B.TILEMIX_EINVAL
    assert lib.tilemix_pack_route_mask(FAKE, 4, 8, FAKE, 0, None) == B.TILEMIX_EINVAL
    assert lib.tilemix_pack_route_mask(None, 4, 8, FAKE, 1, None) == B.TILEMIX_EINVAL
    assert lib.tilemix_pack_route_mask(FAKE, -1, 8, FAKE, 1, None) == B.TILEMIX_EINVAL


def test_workspace_size(lib):
    p = base_params()
    n = ctypes.c_int64(0)
    assert lib.tilemix_prefill_workspace_size(ctypes.byref(p), ctypes.byref(n)) == B.TILEMIX_OK
    # enough for either V path, i.e. the V^T path's: hkv * (ceil(total_k / 64) + batch) tiles of
    # 64 x head_dim fp16 and 256 bytes of work-queue counters (the direct path needs none without
    # an INT8 cache)
    tiles = 2 * (256 // 64 + 1)
    assert n.value == tiles * 64 * 128 * 2 + 256
    p.kv_int8 = 1
    assert lib.tilemix_prefill_workspace_size(ctypes.byref(p), ctypes.byref(n)) == B.TILEMIX_OK
    # + the exact fp16 copy of K8 (total_k x hkv x head_dim); the direct path's K and V copies fit too
    assert n.value == tiles * 64 * 128 * 2 + 256 * 2 * 128 * 2 + 256
    assert n.value >= 2 * 256 * 2 * 128 * 2
    p.head_dim = 80
    assert lib.tilemix_prefill_workspace_size(ctypes.byref(p), ctypes.byref(n)) == B.TILEMIX_EUNSUPPORTED
    assert lib.tilemix_prefill_workspace_size(None, ctypes.byref(n)) == B.TILEMIX_EINVAL


def test_v_path_choice(lib):
    """The V path of a prefill call: the forced one, or the library's choice from the sizes (direct
    for short sequences relative to the KV heads, V^T pre-pass for long ones)."""
    def path(L, hq, hkv, causal=True, v_path=0, batch_total=None):
        T = batch_total or L
        return B.tilemix_prefill_v_path(total_q=T, total_k=T, max_seqlen_k=L, hq=hq, hkv=hkv,
                                        causal=causal, v_path=v_path)
    assert path(8192, 32, 32) == 2      # 8k multi-head
    assert path(256, 2, 2) == 2         # tiny
    assert path(32768, 32, 8) == 1      # 32k GQA 4:1
    assert path(131072, 32, 8) == 1     # 128k
    assert path(16384, 28, 4, batch_total=65752) == 1  # the varlen batch
    assert path(8192, 32, 8) == 2 and path(8193, 32, 8) == 1  # the boundary: 16384 pairs per key row
    assert path(16384, 32, 32) == 2 and path(32768, 32, 32) == 1  # and at most 16k keys
    assert path(8192, 32, 8, causal=False) == 1
    assert path(32768, 32, 8, v_path=2) == 2 and path(256, 2, 2, v_path=1) == 1
    assert path(256, 2, 2, v_path=3) == 0
    assert lib.tilemix_prefill_v_path(None) == 0


def test_version(lib):
    assert B.version() >= 100


def decode_params():
    """A valid INT8-cache decode call (GQA 4:2, one query token, 4096 cached keys)."""
    p = base_params()
    p.k = p.v = None
    p.kv_int8 = 1
    p.v8 = p.v_scale = FAKE
    p.total_q, p.max_seqlen_q = 1, 1
    p.total_k = p.max_seqlen_k = 4096
    p.total_mtiles = 1
    p.words_per_row = 1
    return p


DECODE_BAD_CASES = [
    ("fp16 k/v", lambda p: (setattr(p, "kv_int8", 0), setattr(p, "k", FAKE), setattr(p, "v", FAKE)),
     B.TILEMIX_EUNSUPPORTED),
    ("kv_int8 with fp16 k", lambda p: setattr(p, "k", FAKE), B.TILEMIX_EINVAL),
    ("no v8", lambda p: setattr(p, "v8", None), B.TILEMIX_EINVAL),
    ("too many queries", lambda p: setattr(p, "max_seqlen_q", 9), B.TILEMIX_EUNSUPPORTED),
    ("too many rows", lambda p: (setattr(p, "hq", 16), setattr(p, "hkv", 2), setattr(p, "max_seqlen_q", 4)),
     B.TILEMIX_EUNSUPPORTED),
    ("debug dump", lambda p: setattr(p, "debug_s32", FAKE), B.TILEMIX_EINVAL),
    ("sync stages", lambda p: setattr(p, "debug_sync_stages", 1), B.TILEMIX_EINVAL),
    ("fp16 state", lambda p: setattr(p, "state_fp16", 1), B.TILEMIX_EINVAL),
    ("head_dim", lambda p: setattr(p, "head_dim", 96), B.TILEMIX_EUNSUPPORTED),
    ("null workspace", lambda p: setattr(p, "workspace", None), B.TILEMIX_EINVAL),
    ("small workspace", lambda p: setattr(p, "workspace_bytes", 1024), B.TILEMIX_EINVAL),
    ("misaligned workspace", lambda p: setattr(p, "workspace", FAKE + 16), B.TILEMIX_EINVAL),
    ("too many groups", lambda p: setattr(p, "max_seqlen_k", 128 * 65), B.TILEMIX_EINVAL),
]


@pytest.mark.parametrize("name,mutate,status", DECODE_BAD_CASES, ids=[c[0] for c in DECODE_BAD_CASES])
def test_decode_validation(lib, name, mutate, status):
    p = decode_params()
    mutate(p)
    got = lib.tilemix_decode_fwd(ctypes.byref(p), None)
    assert got == status, (name, B.last_error())
    assert B.last_error().startswith("decode_fwd")


def test_decode_null_params(lib):
    assert lib.tilemix_decode_fwd(None, None) == B.TILEMIX_EINVAL
    assert lib.tilemix_decode_fwd_noalloc(None, None) == B.TILEMIX_EINVAL


# the allocation-free decode call validates everything tilemix_decode_fwd does except the workspace
NOALLOC_BAD_CASES = [c for c in DECODE_BAD_CASES if "workspace" not in c[0]]


@pytest.mark.parametrize("name,mutate,status", NOALLOC_BAD_CASES, ids=[c[0] for c in NOALLOC_BAD_CASES])
def test_decode_noalloc_validation(lib, name, mutate, status):
    p = decode_params()
    mutate(p)
    got = lib.tilemix_decode_fwd_noalloc(ctypes.byref(p), None)
    assert got == status, (name, B.last_error())
    assert B.last_error().startswith("decode_fwd_noalloc")


def test_decode_noalloc_rejects_more_than_its_scratch(lib):
    cap = lib.tilemix_decode_noalloc_max_bytes()
    assert cap == 32 << 20
    p = decode_params()
    p.batch = 8000  # 8000 x 2 KV heads x 4 chunks x 2 rows x 132 fp32 = 67.6 MB of partials
    n = ctypes.c_int64(0)
    assert lib.tilemix_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == B.TILEMIX_OK
    assert n.value > cap
    assert lib.tilemix_decode_fwd_noalloc(ctypes.byref(p), None) == B.TILEMIX_EINVAL
    assert "scratch" in B.last_error()


def test_decode_workspace_size(lib):
    p = decode_params()
    n = ctypes.c_int64(0)
    assert lib.tilemix_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == B.TILEMIX_OK
    # batch x hkv x ceil(4096 / 1024) chunks x (hq / hkv) * max_seqlen_q rows x (head_dim + 4) fp32
    assert n.value == 1 * 2 * 4 * 2 * (128 + 4) * 4
    p.max_seqlen_q = 0
    assert lib.tilemix_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == B.TILEMIX_OK
    assert n.value == 0
    p.head_dim = 80
    assert lib.tilemix_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == B.TILEMIX_EUNSUPPORTED
    p.head_dim, p.hkv = 128, 3
    assert lib.tilemix_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == B.TILEMIX_EINVAL
    assert lib.tilemix_decode_workspace_size(None, ctypes.byref(n)) == B.TILEMIX_EINVAL


def test_route_struct_matches_c_layout(tmp_path):
    fields = [f for f, _ in B.RouteParams._fields_]
    src = tmp_path / "route_layout.c"
    body = "\n".join(f'  printf("%s %zu\\n", "{f}", offsetof(tilemix_route_params, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "tilemix.h"\nint main(void){\n'
                   '  printf("sizeof %zu\\n", sizeof(tilemix_route_params));\n' + body + "\n  return 0;\n}\n")
    exe = tmp_path / "route_layout"
    subprocess.check_call(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = dict(line.split() for line in subprocess.check_output([str(exe)], text=True).splitlines())
    assert int(got["sizeof"]) == ctypes.sizeof(B.RouteParams)
    for f in fields:
        assert int(got[f]) == getattr(B.RouteParams, f).offset, f


def route_params(kv_int8=False):
    """A valid top-k routing call: 2 sequences, 2 KV heads, 4096 keys, 64 x 2 key groups."""
    p = B.RouteParams()
    p.struct_size = ctypes.sizeof(B.RouteParams)
    p.batch, p.hkv, p.head_dim = 2, 2, 128
    p.max_seqlen_k = 4096
    p.cu_seqlens_k = p.cu_mtiles = FAKE
    p.total_mtiles = 40
    p.route_block_n, p.route_group = 64, 2
    p.fp16_per_mille = 100
    if kv_int8:
        p.k8 = p.k_scale = FAKE
        p.kv_int8 = 1
        p.total_k = 6000
    else:
        p.k = FAKE
        p.k_stride_tok, p.k_stride_head = 256, 128
    p.route_words = FAKE
    p.words_per_row = 1
    p.workspace = FAKE
    p.workspace_bytes = 1 << 20
    return p


ROUTE_BAD_CASES = [
    ("struct_size", lambda p: setattr(p, "struct_size", 4), B.TILEMIX_EINVAL),
    ("batch", lambda p: setattr(p, "batch", 0), B.TILEMIX_EINVAL),
    ("hkv", lambda p: setattr(p, "hkv", 70000), B.TILEMIX_EINVAL),
    ("route_block_n", lambda p: setattr(p, "route_block_n", 32), B.TILEMIX_EINVAL),
    ("route_group", lambda p: setattr(p, "route_group", 0), B.TILEMIX_EINVAL),
    ("budget high", lambda p: setattr(p, "fp16_per_mille", 1001), B.TILEMIX_EINVAL),
    ("budget negative", lambda p: setattr(p, "fp16_per_mille", -1), B.TILEMIX_EINVAL),
    ("too many groups", lambda p: setattr(p, "max_seqlen_k", 128 * 65), B.TILEMIX_EINVAL),
    ("null words", lambda p: setattr(p, "route_words", None), B.TILEMIX_EINVAL),
    ("misaligned words", lambda p: setattr(p, "route_words", FAKE + 4), B.TILEMIX_EINVAL),
    ("null cu", lambda p: setattr(p, "cu_mtiles", None), B.TILEMIX_EINVAL),
]

TOPK_BAD_CASES = ROUTE_BAD_CASES + [
    ("head_dim", lambda p: setattr(p, "head_dim", 96), B.TILEMIX_EUNSUPPORTED),
    ("groups past LDS", lambda p: (setattr(p, "max_seqlen_k", 64 * 2 * 8193), setattr(p, "words_per_row", 129)),
     B.TILEMIX_EUNSUPPORTED),
    ("k and k8", lambda p: setattr(p, "k8", FAKE), B.TILEMIX_EINVAL),
    ("no keys", lambda p: setattr(p, "k", None), B.TILEMIX_EINVAL),
    ("odd stride", lambda p: setattr(p, "k_stride_tok", 100), B.TILEMIX_EINVAL),
    ("misaligned k", lambda p: setattr(p, "k", FAKE + 8), B.TILEMIX_EINVAL),
    ("null workspace", lambda p: setattr(p, "workspace", None), B.TILEMIX_EINVAL),
    ("small workspace", lambda p: setattr(p, "workspace_bytes", 64), B.TILEMIX_EINVAL),
    ("misaligned workspace", lambda p: setattr(p, "workspace", FAKE + 64), B.TILEMIX_EINVAL),
]


@pytest.mark.parametrize("name,mutate,status", TOPK_BAD_CASES, ids=[c[0] for c in TOPK_BAD_CASES])
def test_route_topk_validation(lib, name, mutate, status):
    p = route_params()
    mutate(p)
    assert lib.tilemix_route_topk_maxabs(ctypes.byref(p), None) == status, (name, B.last_error())
    assert B.last_error().startswith("route_topk_maxabs")


def test_route_topk_int8_cache_validation(lib):
    for mutate in (lambda p: setattr(p, "k", FAKE), lambda p: setattr(p, "k_scale", None),
                   lambda p: setattr(p, "k8", FAKE + 8), lambda p: setattr(p, "total_k", -1)):
        p = route_params(kv_int8=True)
        mutate(p)
        assert lib.tilemix_route_topk_maxabs(ctypes.byref(p), None) == B.TILEMIX_EINVAL, B.last_error()


@pytest.mark.parametrize("name,mutate,status", ROUTE_BAD_CASES, ids=[c[0] for c in ROUTE_BAD_CASES])
def test_route_bernoulli_validation(lib, name, mutate, status):
    p = route_params()
    p.k = None  # the Bernoulli policy reads no keys and no workspace
    p.workspace = None
    mutate(p)
    assert lib.tilemix_route_bernoulli(ctypes.byref(p), None) == status, (name, B.last_error())
    assert B.last_error().startswith("route_bernoulli")


def test_route_null_params_and_workspace_size(lib):
    assert lib.tilemix_route_topk_maxabs(None, None) == B.TILEMIX_EINVAL
    assert lib.tilemix_route_bernoulli(None, None) == B.TILEMIX_EINVAL
    p = route_params()
    n = ctypes.c_int64(0)
    assert lib.tilemix_route_workspace_size(ctypes.byref(p), ctypes.byref(n)) == B.TILEMIX_OK
    # 4 bytes x batch 2 x hkv 2 x ceil(4096 / 128) groups, rounded up to 256
    assert n.value == 512
    p.max_seqlen_k = 0
    assert lib.tilemix_route_workspace_size(ctypes.byref(p), ctypes.byref(n)) == B.TILEMIX_OK
    assert n.value == 0
    p.route_group = 0
    assert lib.tilemix_route_workspace_size(ctypes.byref(p), ctypes.byref(n)) == B.TILEMIX_EINVAL
    assert lib.tilemix_route_workspace_size(None, ctypes.byref(n)) == B.TILEMIX_EINVAL


QB_BAD = [
    ("head_dim", dict(head_dim=96), B.TILEMIX_EUNSUPPORTED),
    ("block_rows", dict(block_rows=0), B.TILEMIX_EINVAL),
    ("n_head", dict(n_head=0), B.TILEMIX_EINVAL),
    ("batch", dict(batch=0), B.TILEMIX_EINVAL),
    ("negative tokens", dict(n_tok=-1), B.TILEMIX_EINVAL),
    ("null x", dict(x=None), B.TILEMIX_EINVAL),
    ("null cu", dict(cu=None), B.TILEMIX_EINVAL),
    ("null scale", dict(scale=None), B.TILEMIX_EINVAL),
    ("odd stride", dict(stride_tok=100), B.TILEMIX_EINVAL),
    ("misaligned x", dict(x=FAKE + 8), B.TILEMIX_EINVAL),
    ("misaligned x8", dict(x8=FAKE + 4), B.TILEMIX_EINVAL),
]


@pytest.mark.parametrize("name,change,status", QB_BAD, ids=[c[0] for c in QB_BAD])
def test_quantize_blocks_validation(lib, name, change, status):
    a = dict(x=FAKE, n_tok=1000, n_head=4, stride_tok=512, stride_head=128, cu=FAKE, batch=2,
             max_seqlen=600, block_rows=64, x8=FAKE, scale=FAKE, head_dim=128)
    a.update(change)
    got = lib.tilemix_quantize_blocks(a["x"], a["n_tok"], a["n_head"], a["stride_tok"], a["stride_head"],
                                      a["cu"], a["batch"], a["max_seqlen"], a["block_rows"], a["x8"],
                                      a["scale"], a["head_dim"], None)
    assert got == status, (name, B.last_error())
    assert B.last_error().startswith("quantize_blocks")
