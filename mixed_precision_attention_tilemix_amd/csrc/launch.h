// Host-side launchers of the libtilemix kernels (internal; the public ABI is include/tilemix.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tilemix {

// Per-token symmetric INT8 quantization of n_tok x n_head rows of head_dim fp16 values.
hipError_t launch_quantize(const void* x, int64_t n_tok, int32_t n_head, int64_t stride_tok,
                           int64_t stride_head, int8_t* x8, float* scale, int32_t head_dim,
                           hipStream_t stream);

// Block-wise variant: one scale per block of block_rows tokens of one sequence and head, written
// to every row of the block ([n_head, n_tok] layout as above).
hipError_t launch_quantize_blocks(const void* x, int64_t n_tok, int32_t n_head, int64_t stride_tok,
                                  int64_t stride_head, const int32_t* cu, int32_t batch,
                                  int32_t max_seqlen, int32_t block_rows, int8_t* x8, float* scale,
                                  int32_t head_dim, hipStream_t stream);

hipError_t launch_pack(const uint8_t* route, int64_t rows, int32_t t_mask, uint64_t* words,
                       int32_t words_per_row, hipStream_t stream);

// Everything the fused kernel reads, by value.
struct FwdArgs {
  int32_t hq, hkv;
  int64_t total_q, total_k;
  int32_t max_seqlen_q;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* cu_mtiles;
  int32_t total_mtiles;
  const _Float16* q;
  int64_t q_stride_tok, q_stride_head;
  const _Float16* k;
  int64_t k_stride_tok, k_stride_head;
  const _Float16* v;
  int64_t v_stride_tok, v_stride_head;
  const int8_t* q8;
  const float* q_scale;
  const int8_t* k8;
  const float* k_scale;
  const int8_t* v8;
  const float* v_scale;
  const uint64_t* words;
  int32_t wpr, bm_r, bn_r, group;
  int32_t causal;
  float scale_log2;  // softmax_scale * log2(e)
  void* out;
  int32_t out_f32;
  float* lse;
  int32_t* dump;
  int32_t dump_head, dump_m0, dump_mcount, dump_ntiles;
  // workspace written by a pre-pass and read by the fused kernel
  _Float16* vt_ws;        // V^T path: [hkv][vt_tiles][D][64] swizzled V^T tiles
  const _Float16* vt;     // the same, read-only view
  int64_t vt_tiles;       // tile slots per KV head (>= tiles of all sequences)
  _Float16* k16_ws;       // INT8 cache: exact fp16(k8) [total_k, hkv, D], read as k
  _Float16* v16_ws;       // INT8 cache on the direct V path: fp16(v_scale * v8) [total_k, hkv, D], read as v
  int32_t v_direct;       // V rows staged as they are (else V^T tiles from the pre-pass)
  int32_t* sched;         // V^T path: 8 work-queue counters, zeroed by the pre-pass (persistent
                          // launch of the fused kernel); NULL: one workgroup per work item
  int32_t k_block;        // > 0: K scales constant over 64-key tiles (one factor per tile)
  int32_t sync_stages;    // debug instance: every staging load waited for before any compute
  int32_t state_fp16;     // online-softmax state (m, l, O) rounded to binary16 after every key tile
};

// V^T path: V^T tiles (and, with an INT8 cache, fp16 K) into the workspace; must precede
// launch_prefill.
hipError_t launch_vt_pack(const FwdArgs& a, int32_t batch, int32_t max_seqlen_k, int32_t head_dim,
                          bool kv_int8, hipStream_t stream);

// Direct V path with an INT8 cache: exact fp16 K and dequantized fp16 V into the workspace; must
// precede launch_prefill.
hipError_t launch_cache_widen(const FwdArgs& a, int32_t head_dim, hipStream_t stream);

hipError_t launch_prefill(const FwdArgs& a, int32_t batch, int32_t head_dim, bool kv_int8,
                          hipStream_t stream);

// Decode over an INT8 K/V cache: keys per chunk workgroup, and the largest number of query rows
// (query heads per KV head x query tokens) one (sequence, KV head) may carry.
constexpr int kDecodeChunk = 1024;
constexpr int kDecodeMaxRows = 16;

struct DecodeArgs {
  FwdArgs f;          // shapes, inputs, route words and outputs (the prefill workspace fields unused)
  float* part;        // workspace [batch][hkv][nchunk][rmax][head_dim + 4]: per chunk m, l, 2 pad, O
  int32_t nchunk;     // chunks per sequence: ceil(max_seqlen_k / kDecodeChunk)
  int32_t rmax;       // (hq / hkv) * max_seqlen_q
};

// Chunk pass then merge pass, both on `stream`.
hipError_t launch_decode(const DecodeArgs& a, int32_t batch, int32_t head_dim, hipStream_t stream);

// Bytes of the library's own per-device decode scratch (the allocation-free decode entry point
// keeps the per-chunk partials there instead of in a caller workspace).
constexpr int64_t kDecodeScratchBytes = int64_t{32} << 20;

// Device address of that scratch on the current device: looked up once per device with the
// device current, then cached. Allocates nothing.
hipError_t decode_scratch(float** ptr);

// Routing policies fused with packing. Groups per sequence are at most kRouteMaxGroups for the
// top-k policy (its select pass ranks them in LDS).
constexpr int kRouteMaxGroups = 8192;

struct RouteArgs {
  int32_t batch, hkv;
  const int32_t* cu_k;
  const int32_t* cu_mtiles;
  int32_t total_mtiles;
  int64_t span;          // keys per routing group: BN_r * g
  int32_t tmax;          // ceil(max_seqlen_k / span): group slots per (sequence, KV head)
  int32_t per_mille;     // FP16 budget
  const uint16_t* k;     // fp16 bits, or NULL with the INT8 cache
  int64_t k_stride_tok, k_stride_head;
  const int8_t* k8;      // [total_k, hkv, D]
  const float* k_scale;  // [hkv, total_k]
  int64_t total_k;
  uint32_t seed_lo, seed_hi;
  uint64_t thr;          // Bernoulli: FP16 iff Philox word < thr
  uint64_t* words;       // [hkv, total_mtiles, wpr]
  int32_t wpr;
  float* gmax;           // top-k workspace [batch][hkv][tmax]
};

hipError_t launch_route_topk(const RouteArgs& a, int32_t head_dim, bool kv_int8, hipStream_t stream);
hipError_t launch_route_bernoulli(const RouteArgs& a, hipStream_t stream);

}  // namespace tilemix
