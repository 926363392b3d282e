// C ABI of libtilemix (declared in include/tilemix.h): host-side argument validation, the
// thread-local error string and the kernel launches. No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/tilemix.h"
#include "launch.h"
#include "tile_layout.h"

namespace {

thread_local std::string g_last_error;

tilemix_status fail(tilemix_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

tilemix_status ok() {
  g_last_error.clear();
  return TILEMIX_OK;
}

tilemix_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(TILEMIX_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

tilemix_status check_quant_group(const char* name, const void* x, int64_t n, int32_t h,
                                 int64_t st_tok, int64_t st_head, const int8_t* x8,
                                 const float* s, int32_t d) {
  if (x == nullptr && x8 == nullptr && s == nullptr) return TILEMIX_OK;
  if (x == nullptr || x8 == nullptr || s == nullptr)
    return fail(TILEMIX_EINVAL, "quantize_qk: %s input and both outputs must be all set or all NULL", name);
  if (n < 0 || h < 1 || h > 65535)
    return fail(TILEMIX_EINVAL, "quantize_qk: %s has n_tok=%lld heads=%d (heads 1 .. 65535)", name, (long long)n, h);
  if (st_tok < 0 || st_head < 0 || st_tok % 8 || st_head % 8)
    return fail(TILEMIX_EINVAL, "quantize_qk: %s strides must be non-negative multiples of 8 elements", name);
  if (!aligned(x, 16) || !aligned(x8, 8) || !aligned(s, 4))
    return fail(TILEMIX_EINVAL, "quantize_qk: %s pointers misaligned (need 16/8/4 bytes)", name);
  (void)d;
  return TILEMIX_OK;
}

struct WorkspaceLayout {
  int64_t vt_tiles;   // V^T path: V^T tile slots per KV head
  int64_t k16_off;    // INT8 cache: byte offset of the exact fp16 K copy
  int64_t v16_off;    // INT8 cache on the direct V path: byte offset of the dequantized fp16 V
  int64_t sched_off;  // V^T path: byte offset of the fused kernel's 8 work-queue counters
  int64_t total;      // bytes in all
};

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// V^T path: the V^T tiles, then (INT8 cache) the fp16 K copy, then 256 bytes for the fused
// kernel's work-queue counters. Direct path: nothing, or (INT8 cache) the fp16 K copy and the
// dequantized V. The V^T path never needs less.
WorkspaceLayout workspace_layout(const tilemix_fwd_params* p, bool v_direct) {
  WorkspaceLayout w{};
  const int64_t copy = p->kv_int8 ? round_up(p->total_k * p->hkv * p->head_dim * 2, 256) : 0;
  if (v_direct) {
    w.k16_off = 0;
    w.v16_off = copy;
    w.total = 2 * copy;
  } else {
    w.vt_tiles = tilemix::key_tiles_bound(p->total_k, p->batch);
    w.k16_off = round_up(static_cast<int64_t>(p->hkv) * w.vt_tiles * tilemix::kKeyTile * p->head_dim * 2, 256);
    w.sched_off = w.k16_off + copy;
    w.total = w.sched_off + 256;
  }
  return w;
}

// Which V path a call takes. The V^T pre-pass reads and writes V once (about 4 bytes per key
// row and channel) and lets the fused kernel run persistent (its work queues are zeroed by the
// pre-pass); the direct path instead doubles the kernel's LDS reads of V, a cost that grows with
// the work per key. The direct path wins while the work per key row (query-key pairs x query
// heads / (keys x KV heads), estimated from the largest sequence) stays at or under 16384 and the
// sequences are at most 16k keys long. Measured (fused call, direct / V^T): four 4k multi-head
// sequences 0.89, 8k multi-head 0.94, 8k GQA 4:1 0.98, 16k multi-head 1.00, 32k multi-head 1.01,
// 16k GQA 4:1 1.01, 32k GQA 4:1 1.03, the 64k varlen batch 1.02.
bool choose_v_direct(const tilemix_fwd_params* p) {
  if (p->v_path != 0) return p->v_path == 2;
  const double pairs = static_cast<double>(p->total_q) * p->max_seqlen_k * (p->causal ? 0.5 : 1.0);
  return p->max_seqlen_k <= 16384 && pairs * p->hq <= 16384.0 * static_cast<double>(p->total_k) * p->hkv;
}

// Bytes of the decode workspace: per (sequence, KV head, key chunk, query row) the chunk's max,
// sum and unnormalised output.
int64_t decode_workspace(const tilemix_fwd_params* p) {
  const int64_t nchunk = ceil_div(p->max_seqlen_k, tilemix::kDecodeChunk);
  const int64_t rmax = static_cast<int64_t>(p->hq / p->hkv) * p->max_seqlen_q;
  return round_up(static_cast<int64_t>(p->batch) * p->hkv * nchunk * rmax * (p->head_dim + 4) * 4, 256);
}

// The kernel-side view of the shapes, inputs, route words and outputs of a call.
tilemix::FwdArgs fwd_args(const tilemix_fwd_params* p) {
  const float scale = p->softmax_scale > 0.0f ? p->softmax_scale
                                              : 1.0f / std::sqrt(static_cast<float>(p->head_dim));
  tilemix::FwdArgs a{};
  a.hq = p->hq;
  a.hkv = p->hkv;
  a.total_q = p->total_q;
  a.total_k = p->total_k;
  a.max_seqlen_q = p->max_seqlen_q;
  a.cu_q = p->cu_seqlens_q;
  a.cu_k = p->cu_seqlens_k;
  a.cu_mtiles = p->cu_mtiles;
  a.total_mtiles = p->total_mtiles;
  a.q = static_cast<const _Float16*>(p->q);
  a.q_stride_tok = p->q_stride_tok;
  a.q_stride_head = p->q_stride_head;
  a.k = static_cast<const _Float16*>(p->k);
  a.k_stride_tok = p->k_stride_tok;
  a.k_stride_head = p->k_stride_head;
  a.v = static_cast<const _Float16*>(p->v);
  a.v_stride_tok = p->v_stride_tok;
  a.v_stride_head = p->v_stride_head;
  a.q8 = p->q8;
  a.q_scale = p->q_scale;
  a.k8 = p->k8;
  a.k_scale = p->k_scale;
  a.v8 = p->v8;
  a.v_scale = p->v_scale;
  a.words = p->route_words;
  a.wpr = p->words_per_row;
  a.bm_r = p->route_block_m;
  a.bn_r = p->route_block_n;
  a.group = p->route_group;
  a.causal = p->causal ? 1 : 0;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = p->out;
  a.out_f32 = p->out_dtype == 1;
  a.lse = p->lse;
  a.dump = p->debug_s32;
  a.dump_head = p->debug_head;
  a.dump_m0 = p->debug_mtile_begin;
  a.dump_mcount = p->debug_mtile_count;
  a.dump_ntiles = p->debug_ntiles_max;
  a.k_block = p->k_scale_block;
  a.sync_stages = p->debug_sync_stages != 0;
  a.state_fp16 = p->state_fp16 != 0;
  return a;
}

tilemix_status check_params(const tilemix_fwd_params* p, const char* fn) {
  if (p == nullptr) return fail(TILEMIX_EINVAL, "%s: NULL params", fn);
  if (p->struct_size != sizeof(tilemix_fwd_params))
    return fail(TILEMIX_EINVAL, "%s: struct_size %u != %zu", fn, p->struct_size,
                sizeof(tilemix_fwd_params));
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(TILEMIX_EUNSUPPORTED, "%s: head_dim %d (supported: 64, 128)", fn, p->head_dim);
  if (p->batch < 1 || p->hq < 1 || p->hkv < 1 || p->hq % p->hkv)
    return fail(TILEMIX_EINVAL, "%s: batch=%d hq=%d hkv=%d (need hq %% hkv == 0)", fn, p->batch,
                p->hq, p->hkv);
  if (p->total_q < 0 || p->total_k < 0 || p->max_seqlen_q < 0 || p->max_seqlen_k < 0 ||
      p->total_mtiles < 0)
    return fail(TILEMIX_EINVAL, "%s: negative size", fn);
  if (p->route_block_m < 32 || p->route_block_m % 32)
    return fail(TILEMIX_EINVAL, "%s: route_block_m %d is not a positive multiple of 32", fn,
                p->route_block_m);
  if (p->route_block_n < 64 || p->route_block_n % 64)
    return fail(TILEMIX_EINVAL, "%s: route_block_n %d is not a positive multiple of 64", fn,
                p->route_block_n);
  if (p->route_group < 1) return fail(TILEMIX_EINVAL, "%s: route_group %d < 1", fn, p->route_group);
  if (p->words_per_row < 1) return fail(TILEMIX_EINVAL, "%s: words_per_row < 1", fn);
  const int64_t t_mask = ceil_div(p->max_seqlen_k, static_cast<int64_t>(p->route_block_n) * p->route_group);
  if (t_mask > 64LL * p->words_per_row)
    return fail(TILEMIX_EINVAL, "%s: %lld key-tile groups need more than %d words per row", fn,
                (long long)t_mask, p->words_per_row);
  if (!p->cu_seqlens_q || !p->cu_seqlens_k || !p->cu_mtiles || !p->q || !p->k8 || !p->k_scale ||
      !p->route_words || !p->out)
    return fail(TILEMIX_EINVAL, "%s: a required pointer is NULL", fn);
  if ((p->q8 == nullptr) != (p->q_scale == nullptr))
    return fail(TILEMIX_EINVAL, "%s: q8 and q_scale are both set (quantize-once) or both NULL (fused Q quantization)", fn);
  if (p->kv_int8) {
    if (p->k || p->v)
      return fail(TILEMIX_EINVAL, "%s: kv_int8 takes K/V from k8/v8; k and v must be NULL", fn);
    if (!p->v8 || !p->v_scale) return fail(TILEMIX_EINVAL, "%s: kv_int8 needs v8 and v_scale", fn);
  } else {
    if (!p->k || !p->v) return fail(TILEMIX_EINVAL, "%s: fp16 k and v are required", fn);
  }
  if (p->out_dtype != 0 && p->out_dtype != 1)
    return fail(TILEMIX_EINVAL, "%s: out_dtype %d (0 = fp16, 1 = fp32)", fn, p->out_dtype);
  // 16-byte vector access of the fp16 / int8 rows
  const int64_t st[6] = {p->q_stride_tok, p->q_stride_head, p->k_stride_tok, p->k_stride_head,
                         p->v_stride_tok, p->v_stride_head};
  for (int i = 0; i < 6; ++i) {
    if (i >= 2 && p->kv_int8) break;
    if (st[i] < 0 || st[i] % 8) return fail(TILEMIX_EINVAL, "%s: fp16 strides must be multiples of 8", fn);
  }
  // the fused kernel addresses up to 64 K / V rows of a tile with 32-bit byte offsets
  if (!p->kv_int8 && (p->k_stride_tok >= (int64_t{1} << 24) || p->v_stride_tok >= (int64_t{1} << 24)))
    return fail(TILEMIX_EINVAL, "%s: k / v token strides must be below 2^24 elements", fn);
  if (!aligned(p->q, 16) || (p->k && !aligned(p->k, 16)) || (p->v && !aligned(p->v, 16)) ||
      (p->q8 && !aligned(p->q8, 16)) || !aligned(p->k8, 16) || (p->v8 && !aligned(p->v8, 16)) ||
      !aligned(p->out, 16) || !aligned(p->k_scale, 4) || (p->v_scale && !aligned(p->v_scale, 4)) ||
      (p->q_scale && !aligned(p->q_scale, 4)))
    return fail(TILEMIX_EINVAL, "%s: tensors must be 16-byte aligned", fn);
  return TILEMIX_OK;
}

// Checks shared by the two routing policies; *tmax = ceil(max_seqlen_k / (BN_r * g)).
tilemix_status check_route(const tilemix_route_params* p, const char* fn, int64_t* tmax) {
  if (p == nullptr) return fail(TILEMIX_EINVAL, "%s: NULL params", fn);
  if (p->struct_size != sizeof(tilemix_route_params))
    return fail(TILEMIX_EINVAL, "%s: struct_size %u != %zu", fn, p->struct_size,
                sizeof(tilemix_route_params));
  if (p->batch < 1 || p->batch > 65535 || p->hkv < 1 || p->hkv > 65535)
    return fail(TILEMIX_EINVAL, "%s: batch=%d hkv=%d (each 1 .. 65535)", fn, p->batch, p->hkv);
  if (p->max_seqlen_k < 0 || p->total_mtiles < 0) return fail(TILEMIX_EINVAL, "%s: negative size", fn);
  if (p->route_block_n < 64 || p->route_block_n % 64)
    return fail(TILEMIX_EINVAL, "%s: route_block_n %d is not a positive multiple of 64", fn, p->route_block_n);
  if (p->route_group < 1) return fail(TILEMIX_EINVAL, "%s: route_group %d < 1", fn, p->route_group);
  if (p->fp16_per_mille < 0 || p->fp16_per_mille > 1000)
    return fail(TILEMIX_EINVAL, "%s: fp16_per_mille %d outside 0 .. 1000", fn, p->fp16_per_mille);
  if (p->words_per_row < 1) return fail(TILEMIX_EINVAL, "%s: words_per_row < 1", fn);
  *tmax = ceil_div(p->max_seqlen_k, static_cast<int64_t>(p->route_block_n) * p->route_group);
  if (*tmax > 64LL * p->words_per_row)
    return fail(TILEMIX_EINVAL, "%s: %lld key-tile groups need more than %d words per row", fn,
                (long long)*tmax, p->words_per_row);
  if (!p->cu_seqlens_k || !p->cu_mtiles || !p->route_words)
    return fail(TILEMIX_EINVAL, "%s: a required pointer is NULL", fn);
  if (!aligned(p->route_words, 8)) return fail(TILEMIX_EINVAL, "%s: route_words misaligned", fn);
  if (static_cast<int64_t>(p->hkv) * p->total_mtiles * p->words_per_row >= (int64_t{1} << 33))
    return fail(TILEMIX_EINVAL, "%s: too many route words", fn);
  return TILEMIX_OK;
}

int64_t route_workspace(const tilemix_route_params* p) {
  const int64_t tmax = ceil_div(p->max_seqlen_k, static_cast<int64_t>(p->route_block_n) * p->route_group);
  return round_up(int64_t{4} * p->batch * p->hkv * tmax, 256);
}

tilemix::RouteArgs route_args(const tilemix_route_params* p, int64_t tmax) {
  tilemix::RouteArgs a{};
  a.batch = p->batch;
  a.hkv = p->hkv;
  a.cu_k = p->cu_seqlens_k;
  a.cu_mtiles = p->cu_mtiles;
  a.total_mtiles = p->total_mtiles;
  a.span = static_cast<int64_t>(p->route_block_n) * p->route_group;
  a.tmax = static_cast<int32_t>(tmax);
  a.per_mille = p->fp16_per_mille;
  a.k = static_cast<const uint16_t*>(p->k);
  a.k_stride_tok = p->k_stride_tok;
  a.k_stride_head = p->k_stride_head;
  a.k8 = p->k8;
  a.k_scale = p->k_scale;
  a.total_k = p->total_k;
  a.seed_lo = static_cast<uint32_t>(p->seed);
  a.seed_hi = static_cast<uint32_t>(p->seed >> 32);
  a.thr = (static_cast<uint64_t>(p->fp16_per_mille) << 32) / 1000;
  a.words = p->route_words;
  a.wpr = p->words_per_row;
  a.gmax = static_cast<float*>(p->workspace);
  return a;
}

// Checks shared by both decode entry points (everything except the workspace).
tilemix_status check_decode(const tilemix_fwd_params* p, const char* what) {
  if (tilemix_status st = check_params(p, what)) return st;
  if (!p->kv_int8) return fail(TILEMIX_EUNSUPPORTED, "%s: reads an INT8 K/V cache (kv_int8 = 1)", what);
  if (p->max_seqlen_q > 8)
    return fail(TILEMIX_EUNSUPPORTED, "%s: max_seqlen_q %d > 8 (use tilemix_prefill_fwd)", what, p->max_seqlen_q);
  if ((p->hq / p->hkv) * p->max_seqlen_q > tilemix::kDecodeMaxRows)
    return fail(TILEMIX_EUNSUPPORTED, "%s: (hq / hkv) * max_seqlen_q = %d > %d query rows per KV head", what,
                (p->hq / p->hkv) * p->max_seqlen_q, tilemix::kDecodeMaxRows);
  if (p->debug_s32) return fail(TILEMIX_EINVAL, "%s: the debug dump is a prefill feature", what);
  if (p->debug_sync_stages || p->state_fp16)
    return fail(TILEMIX_EINVAL, "%s: debug_sync_stages and state_fp16 are prefill features", what);
  return TILEMIX_OK;
}

tilemix_status launch_decode_into(const tilemix_fwd_params* p, float* part, void* stream, const char* what) {
  tilemix::DecodeArgs d{};
  d.f = fwd_args(p);
  d.part = part;
  d.nchunk = static_cast<int32_t>(ceil_div(p->max_seqlen_k, tilemix::kDecodeChunk));
  d.rmax = (p->hq / p->hkv) * p->max_seqlen_q;
  return from_hip(tilemix::launch_decode(d, p->batch, p->head_dim, static_cast<hipStream_t>(stream)), what);
}

}  // namespace

extern "C" {

const char* tilemix_last_error(void) { return g_last_error.c_str(); }

int32_t tilemix_version(void) { return 100; }

tilemix_status tilemix_quantize_qk(const void* q, int64_t total_q, int32_t hq,
                                   int64_t q_stride_tok, int64_t q_stride_head, int8_t* q8,
                                   float* q_scale, const void* k, int64_t total_k, int32_t hk,
                                   int64_t k_stride_tok, int64_t k_stride_head, int8_t* k8,
                                   float* k_scale, int32_t head_dim, void* stream) {
  if (head_dim != 64 && head_dim != 128)
    return fail(TILEMIX_EUNSUPPORTED, "quantize_qk: head_dim %d (supported: 64, 128)", head_dim);
  tilemix_status st;
  if ((st = check_quant_group("q", q, total_q, hq, q_stride_tok, q_stride_head, q8, q_scale, head_dim)))
    return st;
  if ((st = check_quant_group("k", k, total_k, hk, k_stride_tok, k_stride_head, k8, k_scale, head_dim)))
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (q) {
    hipError_t e = tilemix::launch_quantize(q, total_q, hq, q_stride_tok, q_stride_head, q8,
                                            q_scale, head_dim, s);
    if (e != hipSuccess) return from_hip(e, "quantize_qk(q)");
  }
  if (k) {
    hipError_t e = tilemix::launch_quantize(k, total_k, hk, k_stride_tok, k_stride_head, k8,
                                            k_scale, head_dim, s);
    if (e != hipSuccess) return from_hip(e, "quantize_qk(k)");
  }
  return ok();
}

tilemix_status tilemix_quantize_blocks(const void* x, int64_t n_tok, int32_t n_head, int64_t stride_tok,
                                       int64_t stride_head, const int32_t* cu_seqlens, int32_t batch,
                                       int32_t max_seqlen, int32_t block_rows, int8_t* x8, float* scale,
                                       int32_t head_dim, void* stream) {
  if (head_dim != 64 && head_dim != 128)
    return fail(TILEMIX_EUNSUPPORTED, "quantize_blocks: head_dim %d (supported: 64, 128)", head_dim);
  if (n_tok < 0 || n_head < 1 || n_head > 65535 || batch < 1 || batch > 65535 || max_seqlen < 0)
    return fail(TILEMIX_EINVAL, "quantize_blocks: n_tok=%lld n_head=%d batch=%d max_seqlen=%d",
                (long long)n_tok, n_head, batch, max_seqlen);
  if (block_rows < 1) return fail(TILEMIX_EINVAL, "quantize_blocks: block_rows %d < 1", block_rows);
  if (!x || !x8 || !scale || !cu_seqlens) return fail(TILEMIX_EINVAL, "quantize_blocks: NULL pointer");
  if (stride_tok < 0 || stride_head < 0 || stride_tok % 8 || stride_head % 8)
    return fail(TILEMIX_EINVAL, "quantize_blocks: strides must be non-negative multiples of 8 elements");
  if (!aligned(x, 16) || !aligned(x8, 8) || !aligned(scale, 4))
    return fail(TILEMIX_EINVAL, "quantize_blocks: pointers misaligned (need 16/8/4 bytes)");
  return from_hip(tilemix::launch_quantize_blocks(x, n_tok, n_head, stride_tok, stride_head, cu_seqlens, batch,
                                                  max_seqlen, block_rows, x8, scale, head_dim,
                                                  static_cast<hipStream_t>(stream)),
                  "quantize_blocks");
}

tilemix_status tilemix_pack_route_mask(const uint8_t* route, int64_t rows, int32_t t_mask,
                                       uint64_t* words, int32_t words_per_row, void* stream) {
  if (rows < 0 || t_mask < 0) return fail(TILEMIX_EINVAL, "pack_route_mask: negative size");
  if (words_per_row < 1 || static_cast<int64_t>(t_mask) > 64LL * words_per_row)
    return fail(TILEMIX_EINVAL, "pack_route_mask: t_mask %d does not fit %d words per row", t_mask,
                words_per_row);
  if (rows > 0 && (words == nullptr || (t_mask > 0 && route == nullptr)))
    return fail(TILEMIX_EINVAL, "pack_route_mask: NULL route or words");
  if (!aligned(words, 8)) return fail(TILEMIX_EINVAL, "pack_route_mask: words misaligned");
  return from_hip(tilemix::launch_pack(route, rows, t_mask, words, words_per_row,
                                       static_cast<hipStream_t>(stream)),
                  "pack_route_mask");
}

tilemix_status tilemix_prefill_workspace_size(const tilemix_fwd_params* p, int64_t* bytes) {
  if (p == nullptr || bytes == nullptr) return fail(TILEMIX_EINVAL, "prefill_workspace_size: NULL argument");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(TILEMIX_EUNSUPPORTED, "prefill_workspace_size: head_dim %d (supported: 64, 128)", p->head_dim);
  if (p->batch < 1 || p->hkv < 1 || p->total_k < 0)
    return fail(TILEMIX_EINVAL, "prefill_workspace_size: batch=%d hkv=%d total_k=%lld", p->batch, p->hkv,
                (long long)p->total_k);
  *bytes = workspace_layout(p, false).total;  // enough for either V path
  return ok();
}

int32_t tilemix_prefill_v_path(const tilemix_fwd_params* p) {
  if (p == nullptr || p->v_path < 0 || p->v_path > 2) return 0;
  return choose_v_direct(p) ? 2 : 1;
}

tilemix_status tilemix_prefill_fwd(const tilemix_fwd_params* p, void* stream) {
  if (tilemix_status st = check_params(p, "prefill_fwd")) return st;
  if (p->debug_s32) {
    if (p->debug_head < 0 || p->debug_head >= p->hq || p->debug_mtile_begin < 0 ||
        p->debug_mtile_count < 0 || p->debug_mtile_begin + p->debug_mtile_count > p->total_mtiles)
      return fail(TILEMIX_EINVAL, "prefill_fwd: debug head/route-row range out of bounds");
    if (p->debug_ntiles_max < ceil_div(p->max_seqlen_k, p->route_block_n))
      return fail(TILEMIX_EINVAL, "prefill_fwd: debug_ntiles_max %d < ceil(max_seqlen_k / route_block_n)",
                  p->debug_ntiles_max);
  }
  if ((p->debug_s32 != nullptr) + (p->debug_sync_stages != 0) + (p->state_fp16 != 0) > 1)
    return fail(TILEMIX_EINVAL, "prefill_fwd: at most one of debug_s32, debug_sync_stages, state_fp16");
  if (p->k_scale_block < 0 || p->k_scale_block % tilemix::kKeyTile)
    return fail(TILEMIX_EINVAL, "prefill_fwd: k_scale_block %d is not 0 or a multiple of %d", p->k_scale_block,
                tilemix::kKeyTile);
  if (p->v_path < 0 || p->v_path > 2)
    return fail(TILEMIX_EINVAL, "prefill_fwd: v_path %d (0, 1 or 2)", p->v_path);
  const bool v_direct = choose_v_direct(p);
  const WorkspaceLayout ws = workspace_layout(p, v_direct);
  if (ws.total > 0 && (p->workspace == nullptr || !aligned(p->workspace, 256) || p->workspace_bytes < ws.total))
    return fail(TILEMIX_EINVAL, "prefill_fwd: workspace must be 256-byte aligned and hold %lld bytes (got %lld)",
                (long long)ws.total, (long long)p->workspace_bytes);
  if (p->total_q == 0 || p->max_seqlen_q == 0) return ok();

  tilemix::FwdArgs a = fwd_args(p);
  hipStream_t s = static_cast<hipStream_t>(stream);
  a.v_direct = v_direct ? 1 : 0;
  char* ws_base = static_cast<char*>(p->workspace);
  if (p->kv_int8) {  // the FP16-routed tiles read the exact fp16 copy of K8
    a.k16_ws = reinterpret_cast<_Float16*>(ws_base + ws.k16_off);
    a.k = a.k16_ws;
    a.k_stride_tok = static_cast<int64_t>(p->hkv) * p->head_dim;
    a.k_stride_head = p->head_dim;
  }
  hipError_t e = hipSuccess;
  if (v_direct) {
    if (p->kv_int8) {  // P.V reads the dequantized copy of V8
      a.v16_ws = reinterpret_cast<_Float16*>(ws_base + ws.v16_off);
      a.v = a.v16_ws;
      a.v_stride_tok = static_cast<int64_t>(p->hkv) * p->head_dim;
      a.v_stride_head = p->head_dim;
      e = tilemix::launch_cache_widen(a, p->head_dim, s);
    }
  } else {
    a.vt_ws = reinterpret_cast<_Float16*>(ws_base);
    a.vt = a.vt_ws;
    a.vt_tiles = ws.vt_tiles;
    // the pre-pass zeroes the counters of the fused kernel's persistent launch (it runs whenever
    // there is a key; without one the fused kernel takes one workgroup per work item)
    if (p->max_seqlen_k > 0) a.sched = reinterpret_cast<int32_t*>(ws_base + ws.sched_off);
    e = tilemix::launch_vt_pack(a, p->batch, p->max_seqlen_k, p->head_dim, p->kv_int8 != 0, s);
  }
  if (e != hipSuccess) return from_hip(e, "prefill_fwd (pre-pass)");
  return from_hip(tilemix::launch_prefill(a, p->batch, p->head_dim, p->kv_int8 != 0, s), "prefill_fwd");
}

tilemix_status tilemix_decode_workspace_size(const tilemix_fwd_params* p, int64_t* bytes) {
  if (p == nullptr || bytes == nullptr) return fail(TILEMIX_EINVAL, "decode_workspace_size: NULL argument");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(TILEMIX_EUNSUPPORTED, "decode_workspace_size: head_dim %d (supported: 64, 128)", p->head_dim);
  if (p->batch < 1 || p->hq < 1 || p->hkv < 1 || p->hq % p->hkv || p->max_seqlen_q < 0 ||
      p->max_seqlen_k < 0)
    return fail(TILEMIX_EINVAL, "decode_workspace_size: batch=%d hq=%d hkv=%d max_seqlen_q=%d max_seqlen_k=%d",
                p->batch, p->hq, p->hkv, p->max_seqlen_q, p->max_seqlen_k);
  *bytes = decode_workspace(p);
  return ok();
}

tilemix_status tilemix_decode_fwd(const tilemix_fwd_params* p, void* stream) {
  if (tilemix_status st = check_decode(p, "decode_fwd")) return st;
  const int64_t need = decode_workspace(p);
  if (need > 0 && (p->workspace == nullptr || !aligned(p->workspace, 256) || p->workspace_bytes < need))
    return fail(TILEMIX_EINVAL, "decode_fwd: workspace must be 256-byte aligned and hold %lld bytes (got %lld)",
                (long long)need, (long long)p->workspace_bytes);
  if (p->total_q == 0 || p->max_seqlen_q == 0) return ok();
  return launch_decode_into(p, static_cast<float*>(p->workspace), stream, "decode_fwd");
}

int64_t tilemix_decode_noalloc_max_bytes(void) { return tilemix::kDecodeScratchBytes; }

tilemix_status tilemix_decode_fwd_noalloc(const tilemix_fwd_params* p, void* stream) {
  if (tilemix_status st = check_decode(p, "decode_fwd_noalloc")) return st;
  const int64_t need = decode_workspace(p);
  if (need > tilemix::kDecodeScratchBytes)
    return fail(TILEMIX_EINVAL,
                "decode_fwd_noalloc: these shapes need %lld bytes of decode scratch, more than the library's "
                "%lld (use tilemix_decode_fwd with a workspace)",
                (long long)need, (long long)tilemix::kDecodeScratchBytes);
  if (p->total_q == 0 || p->max_seqlen_q == 0) return ok();
  float* part = nullptr;
  if (hipError_t e = tilemix::decode_scratch(&part); e != hipSuccess)
    return from_hip(e, "decode_fwd_noalloc (scratch address)");
  return launch_decode_into(p, part, stream, "decode_fwd_noalloc");
}

tilemix_status tilemix_route_workspace_size(const tilemix_route_params* p, int64_t* bytes) {
  if (p == nullptr || bytes == nullptr) return fail(TILEMIX_EINVAL, "route_workspace_size: NULL argument");
  if (p->batch < 1 || p->hkv < 1 || p->max_seqlen_k < 0 || p->route_block_n < 1 || p->route_group < 1)
    return fail(TILEMIX_EINVAL, "route_workspace_size: batch=%d hkv=%d max_seqlen_k=%d route_block_n=%d route_group=%d",
                p->batch, p->hkv, p->max_seqlen_k, p->route_block_n, p->route_group);
  *bytes = route_workspace(p);
  return ok();
}

tilemix_status tilemix_route_topk_maxabs(const tilemix_route_params* p, void* stream) {
  int64_t tmax = 0;
  if (tilemix_status st = check_route(p, "route_topk_maxabs", &tmax)) return st;
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(TILEMIX_EUNSUPPORTED, "route_topk_maxabs: head_dim %d (supported: 64, 128)", p->head_dim);
  if (tmax > tilemix::kRouteMaxGroups)
    return fail(TILEMIX_EUNSUPPORTED, "route_topk_maxabs: %lld groups per sequence > %d", (long long)tmax,
                tilemix::kRouteMaxGroups);
  if (p->kv_int8) {
    if (p->k || !p->k8 || !p->k_scale)
      return fail(TILEMIX_EINVAL, "route_topk_maxabs: kv_int8 reads k8 and k_scale; k must be NULL");
    if (p->total_k < 0) return fail(TILEMIX_EINVAL, "route_topk_maxabs: negative total_k");
    if (!aligned(p->k8, 16) || !aligned(p->k_scale, 4))
      return fail(TILEMIX_EINVAL, "route_topk_maxabs: k8 / k_scale misaligned (16 / 4 bytes)");
  } else {
    if (!p->k || p->k8 || p->k_scale)
      return fail(TILEMIX_EINVAL, "route_topk_maxabs: fp16 keys are read from k; k8 and k_scale must be NULL");
    if (p->k_stride_tok < 0 || p->k_stride_head < 0 || p->k_stride_tok % 8 || p->k_stride_head % 8)
      return fail(TILEMIX_EINVAL, "route_topk_maxabs: k strides must be non-negative multiples of 8");
    if (!aligned(p->k, 16)) return fail(TILEMIX_EINVAL, "route_topk_maxabs: k must be 16-byte aligned");
  }
  const int64_t need = route_workspace(p);
  if (need > 0 && (p->workspace == nullptr || !aligned(p->workspace, 256) || p->workspace_bytes < need))
    return fail(TILEMIX_EINVAL, "route_topk_maxabs: workspace must be 256-byte aligned and hold %lld bytes (got %lld)",
                (long long)need, (long long)p->workspace_bytes);
  if (p->total_mtiles == 0) return ok();
  return from_hip(tilemix::launch_route_topk(route_args(p, tmax), p->head_dim, p->kv_int8 != 0,
                                             static_cast<hipStream_t>(stream)),
                  "route_topk_maxabs");
}

tilemix_status tilemix_route_bernoulli(const tilemix_route_params* p, void* stream) {
  int64_t tmax = 0;
  if (tilemix_status st = check_route(p, "route_bernoulli", &tmax)) return st;
  return from_hip(tilemix::launch_route_bernoulli(route_args(p, tmax), static_cast<hipStream_t>(stream)),
                  "route_bernoulli");
}

}  // extern "C"
