/*
 * tilemix.h - C ABI of libtilemix.so: tile-group precision-routed fused prefill attention
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one defined in "TileMix: Tile-Centric Mixed-Precision Attention for LLM
 * Inference Acceleration" (arXiv 2608.17336): the L_q x L_k score matrix is cut into route tiles
 * of BM_r x BN_r; a packed bitmask selects, per (KV head, query-tile row, key-tile group), either
 * an FP16 QK^T or an INT8 QK^T with int32 accumulation and per-token scale restoration; both
 * paths feed one online-softmax state (row max, normaliser, output accumulator) before an FP16
 * P.V (Sections 3.1, 4.1-4.3).
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller, including the workspace of
 *     tilemix_prefill_fwd (sized by tilemix_prefill_workspace_size). The library allocates no
 *     device memory and keeps no state other than a thread-local error string.
 *   - Calls are asynchronous: they validate the host-side arguments, enqueue kernels on `stream`
 *     (a hipStream_t; NULL = the null stream) and return. The caller synchronises.
 *     The contents of device arrays (cu_seqlens values, route bits) are not validated; values
 *     that contradict the host-side sizes are undefined behaviour.
 *   - Results are bitwise deterministic run to run (no atomics).
 *   - Token-major layouts: a fp16 or int8 tensor of `n` tokens and `h` heads of `d` channels is
 *     [n, h, d]; fp16 inputs may carry element strides for the token and head dimensions
 *     (channel stride 1). Per-token scales are head-major [h, n] fp32.
 *   - Every call returns TILEMIX_OK or an error status; tilemix_last_error() then describes it.
 */
#ifndef TILEMIX_H
#define TILEMIX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TILEMIX_OK = 0,
  TILEMIX_EINVAL = 1,       /* an argument is out of range, inconsistent or NULL when required */
  TILEMIX_EUNSUPPORTED = 2, /* a valid request outside what the kernels implement (e.g. head_dim) */
  TILEMIX_ELAUNCH = 3       /* a HIP launch error was reported */
} tilemix_status;

/* Text of the last non-OK status returned on the calling thread ("" if none). The pointer stays
 * valid until the next tilemix call on the same thread. */
const char* tilemix_last_error(void);

/* Library version as 10000*major + 100*minor + patch. */
int32_t tilemix_version(void);

/*
 * tilemix_quantize_qk - the quantize-once pass (Section 4.3 "quantize-once mode"; the
 * quantizer psi of Section 3.2 taken per token and per head).
 *
 * For every token t and head h, with x = the head_dim fp16 channels of that row:
 *   a = max_c |x_c|;  a == 0 -> scale = 0, codes = 0;
 *   otherwise inv = 127/a and scale = a/127 (correctly rounded fp32 divisions),
 *   code_c = clamp(rint(x_c * inv), -127, 127)   (fp32 product, round half to even).
 *
 *   q       fp16 [total_q, hq, head_dim] with element strides q_stride_tok / q_stride_head
 *   q8      int8 [total_q, hq, head_dim] contiguous (output)
 *   q_scale fp32 [hq, total_q]            (output)
 * and the same for k / k8 / k_scale with total_k, hk. Either group may be skipped by passing
 * NULL input AND output pointers for it (e.g. only K and V of an INT8 cache, or only Q).
 * head_dim must be 64 or 128 (TILEMIX_EUNSUPPORTED otherwise).
 */
tilemix_status tilemix_quantize_qk(const void* q, int64_t total_q, int32_t hq,
                                   int64_t q_stride_tok, int64_t q_stride_head, int8_t* q8,
                                   float* q_scale, const void* k, int64_t total_k, int32_t hk,
                                   int64_t k_stride_tok, int64_t k_stride_head, int8_t* k8,
                                   float* k_scale, int32_t head_dim, void* stream);

/*
 * tilemix_quantize_blocks - the block-wise form of the quantizer (Section 4.3: Q and K quantized
 * "blockwise" with per-block scales; psi of Section 3.2). A block is block_rows consecutive tokens
 * of one sequence (cu_seqlens, device [batch+1]; the last block of a sequence may be shorter,
 * blocks never straddle sequences) and one head: a = max|x| over its rows and channels, then the
 * per-token quantizer's steps with that a. Every row of the block receives the block's scale, so
 * x8 [n_tok, n_head, d] and scale [n_head, n_tok] have the layouts of tilemix_quantize_qk and feed
 * tilemix_prefill_fwd / tilemix_decode_fwd unchanged (e.g. Q blocks of route_block_m rows and K
 * blocks of route_block_n rows: one scale per route tile row / column). block_rows = 1 gives
 * tilemix_quantize_qk's result. x is fp16 [n_tok, n_head, d] with element strides (multiples of
 * 8, 16-byte aligned). max_seqlen >= every sequence length.
 * Errors: EINVAL for NULL pointers, bad strides / alignment, block_rows < 1, n_head or batch
 * outside 1..65535; EUNSUPPORTED for head_dim other than 64/128.
 */
tilemix_status tilemix_quantize_blocks(const void* x, int64_t n_tok, int32_t n_head, int64_t stride_tok,
                                       int64_t stride_head, const int32_t* cu_seqlens, int32_t batch,
                                       int32_t max_seqlen, int32_t block_rows, int8_t* x8, float* scale,
                                       int32_t head_dim, void* stream);

/*
 * tilemix_pack_route_mask - packs a routing map into bitmask words (Section 4.2, packing and
 * lookup equations: b = sum_j R_j 2^j, R_j = (b >> j) & 1).
 *
 *   route  uint8 [rows, t_mask], each 1 (INT8 path) or 0 (FP16 path); rows = hk * total_mtiles
 *          in the order [h_k][route row].
 *   words  uint64 [rows, words_per_row] (output). Group g lives in word g >> 6 at bit g & 63;
 *          bits at or above t_mask are written 0. words_per_row >= ceil(t_mask / 64).
 * Bytes other than 0/1 in `route` are treated as 1 (any nonzero = INT8).
 */
tilemix_status tilemix_pack_route_mask(const uint8_t* route, int64_t rows, int32_t t_mask,
                                       uint64_t* words, int32_t words_per_row, void* stream);

typedef struct tilemix_fwd_params {
  uint32_t struct_size;         /* sizeof(tilemix_fwd_params) */
  int32_t batch;                /* number of sequences, >= 1 */
  int32_t hq, hkv;              /* query / KV heads; hq % hkv == 0; h_k = h_q / (hq / hkv) */
  int32_t head_dim;             /* 64 or 128 */
  int64_t total_q, total_k;     /* tokens over all sequences */
  int32_t max_seqlen_q;         /* >= every L_q,b (sizes the grid) */
  int32_t max_seqlen_k;         /* >= every L_k,b */
  const int32_t* cu_seqlens_q;  /* device [batch+1], prefix sums of L_q,b */
  const int32_t* cu_seqlens_k;  /* device [batch+1], prefix sums of L_k,b */
  const int32_t* cu_mtiles;     /* device [batch+1], prefix sums of ceil(L_q,b / route_block_m) */
  int32_t total_mtiles;         /* cu_mtiles[batch] */

  const void* q;                /* fp16 [total_q, hq, d] (strided) - FP16 score path */
  int64_t q_stride_tok, q_stride_head;
  const void* k;                /* fp16 [total_k, hkv, d] (strided); NULL iff kv_int8 */
  int64_t k_stride_tok, k_stride_head;
  const void* v;                /* fp16 [total_k, hkv, d] (strided); NULL iff kv_int8 */
  int64_t v_stride_tok, v_stride_head;

  const int8_t* q8;             /* [total_q, hq, d], from tilemix_quantize_qk; or NULL together */
  const float* q_scale;         /* [hq, total_q]     with q_scale: the kernel quantizes Q itself */
  const int8_t* k8;             /* [total_k, hkv, d] */
  const float* k_scale;         /* [hkv, total_k] */
  const int8_t* v8;             /* [total_k, hkv, d]; kv_int8 only (V = v_scale * v8) */
  const float* v_scale;         /* [hkv, total_k];    kv_int8 only */
  int32_t kv_int8;              /* 1: K/V are an INT8 cache (K = k_scale*k8, V = v_scale*v8) */

  const uint64_t* route_words;  /* [hkv, total_mtiles, words_per_row], from pack */
  int32_t words_per_row;        /* >= ceil(T_mask / 64) for every sequence */
  int32_t route_block_m;        /* BM_r: query rows per route tile, multiple of 32 */
  int32_t route_block_n;        /* BN_r: keys per key tile, multiple of 64 */
  int32_t route_group;          /* g >= 1: key tiles per routing bit; g_j = floor(n / g) */

  int32_t causal;               /* 1: key j legal for query i iff j <= i + (L_k - L_q) */
  float softmax_scale;          /* <= 0 selects 1/sqrt(head_dim) */

  void* out;                    /* [total_q, hq, d] contiguous, fp16 or fp32 (output) */
  int32_t out_dtype;            /* 0 = fp16, 1 = fp32 */
  float* lse;                   /* optional [hq, total_q] natural-log sum-exp (output) */

  /* Optional debug dump of the raw int32 accumulators of INT8-routed tiles for one query head:
   * dump[r - debug_mtile_begin][n][ii][jj], shape [debug_mtile_count, debug_ntiles_max,
   * route_block_m, route_block_n], for route rows r in [begin, begin+count) and key tiles n.
   * Every element the kernel computes for an INT8-routed tile is written (masked positions of
   * diagonal tiles included); FP16-routed tiles, skipped tiles and out-of-sequence elements are
   * left untouched, so the caller pre-fills a sentinel. NULL disables it. */
  int32_t* debug_s32;
  int32_t debug_head, debug_mtile_begin, debug_mtile_count, debug_ntiles_max;

  /* Device scratch of at least tilemix_prefill_workspace_size() bytes, 256-byte aligned,
   * owned by the caller; its contents on entry are irrelevant and on return unspecified.
   * It holds the transposed V tiles (and, with kv_int8, an fp16 copy of K8) and, on the V^T
   * path, the fused kernel's work-queue counters. Calls that share one workspace must not
   * overlap in time. */
  void* workspace;
  int64_t workspace_bytes;

  /* 0, or a multiple of 64: the caller guarantees that k_scale is constant over blocks of
   * k_scale_block keys counted from the first key of each sequence (as tilemix_quantize_blocks
   * writes them with block_rows = k_scale_block; the blockwise quantization with per-block
   * scales of Section 4.3). tilemix_prefill_fwd then takes one K scale per 64-key tile (that of
   * its first key) instead of one per key. Any other k_scale content with a nonzero value is
   * undefined. tilemix_decode_fwd ignores it. */
  int32_t k_scale_block;

  /* Nonzero: a single-buffered debug instance of tilemix_prefill_fwd. It loads each key tile
   * into the one LDS stage and waits for the loads before any wavefront computes on it, where the
   * production kernel streams tile n+1 into a second stage while tile n is computed. Its O, LSE
   * equal the production kernel's bit for bit; a difference means a staging race. Slower. At most
   * one of debug_s32, debug_sync_stages and state_fp16 may be set (else TILEMIX_EINVAL);
   * tilemix_decode_fwd rejects it (TILEMIX_EINVAL). */
  int32_t debug_sync_stages;

  /* Nonzero: the FP16-state variant (the TileMix page, Section 4.3 and Appendix G.3): the
   * online-softmax state kept between key tiles (running row max, row sum, output accumulator)
   * is rounded to binary16 after every 64-key tile; scores, P and the accumulation inside a tile
   * stay as without it. The row max is held in log2 units, so |max score| * log2(e) must stay
   * below 65504. 0 keeps fp32 state. Prefill only: tilemix_decode_fwd rejects it. */
  int32_t state_fp16;
  /* How the fused prefill kernel reads V (results are identical either way): 1 = a pre-pass
   * writes V transposed into the workspace, tile by tile; 2 = the kernel stages V rows as they
   * are and transposes them with its LDS reads (no pre-pass, no workspace without kv_int8);
   * 0 = the library chooses (2 when the V pre-pass would be a sizable share of the call: short
   * sequences, at most 16k keys, relative to the number of KV heads; 1 otherwise). Prefill only;
   * decode ignores it. */
  int32_t v_path;
} tilemix_fwd_params;

/*
 * tilemix_prefill_workspace_size - bytes of device workspace tilemix_prefill_fwd needs for
 * these parameters on either V path (only batch, hkv, head_dim, total_k and kv_int8 are read):
 * the V^T path's V^T tiles (plus, with kv_int8, the fp16 copy of K8) and 256 bytes of work-queue
 * counters, which also covers the direct path (none, or with kv_int8 the fp16 copies of K8 and
 * of the dequantized V8). Writes *bytes.
 * Errors: EINVAL for NULL arguments or negative sizes, EUNSUPPORTED for head_dim other than
 * 64/128.
 */
tilemix_status tilemix_prefill_workspace_size(const tilemix_fwd_params* params, int64_t* bytes);

/*
 * tilemix_prefill_v_path - the V path tilemix_prefill_fwd takes for these parameters: 1 (V^T
 * pre-pass) or 2 (direct), i.e. params->v_path when it is 1 or 2, else the library's choice from
 * total_q, total_k, max_seqlen_k, hq, hkv and causal. Returns 0 for NULL or a v_path outside
 * 0..2. Reads nothing on the device.
 */
int32_t tilemix_prefill_v_path(const tilemix_fwd_params* params);

/*
 * tilemix_prefill_fwd - the fused routed attention (Sections 4.1 and 4.3).
 *
 * For each sequence b, query head h_q and query i < L_q,b, with h_k = h_q / (hq/hkv) and
 * key tile n = floor(j / BN_r), group g_j = floor(n / g), route row r = cu_mtiles[b] +
 * floor(i / BM_r) and bit R = (route_words[h_k][r][g_j >> 6] >> (g_j & 63)) & 1:
 *   s_ij = q_scale[h_q][i] * k_scale[h_k][j] * (q8_i . k8_j) * softmax_scale    if R = 1
 *   s_ij = (q_i . K_j) * softmax_scale                                         if R = 0
 * (K_j = fp16 K, or k_scale*k8 with kv_int8), over the legal keys j; then
 * O_i = sum_j softmax(s_i)_j V_j and LSE_i = log sum_j exp(s_ij). A query with no legal key
 * gets O = 0 and LSE = -inf. Scores, softmax state and the P.V accumulator are fp32; P is
 * rounded to fp16 for the FP16 P.V product.
 *
 * Q quantization: with q8 / q_scale set, the INT8 path reads the codes of the quantize-once pass
 * (Section 4.3, "quantize-once mode"). With both NULL the fused kernel quantizes each query row
 * when it loads it, with the same arithmetic as tilemix_quantize_qk (per-token symmetric,
 * bit-identical codes and scales), so the separate Q pass is skipped. One NULL is EINVAL.
 *
 * Implementation: on the V^T path (v_path) a pre-pass writes V^T tiles (and, with kv_int8, fp16
 * K) into the workspace and zeroes the work-queue counters through which the fused kernel's
 * workgroups (as many as the device holds at once) share out the work; on the direct path only
 * kv_int8 has a pre-pass (fp16 K and dequantized V); then the fused kernel runs. All of it is
 * enqueued on `stream`. With no pre-pass (direct path, fp16 K/V) the workspace is not touched
 * and may be NULL.
 *
 * Errors: EINVAL for a NULL required pointer, struct_size mismatch, hq % hkv != 0,
 * route_block_m not a multiple of 32, route_block_n not a multiple of 64, route_group < 1,
 * k_scale_block negative or not a multiple of 64, words_per_row < 1, kv_int8 with non-NULL
 * k/v (or without v8/v_scale), fp16 strides not multiples of 8 or k / v token strides of 2^24
 * elements or more, v_path outside 0..2, a bad debug range, a misaligned or too small workspace
 * (or a NULL one where the V path needs one); EUNSUPPORTED for head_dim other than 64/128.
 */
tilemix_status tilemix_prefill_fwd(const tilemix_fwd_params* params, void* stream);

/*
 * tilemix_decode_workspace_size - bytes of device workspace tilemix_decode_fwd needs for these
 * parameters (batch, hq, hkv, head_dim, max_seqlen_q and max_seqlen_k are read). Writes *bytes
 * (0 when there is nothing to compute). Errors: EINVAL for NULL arguments, hq % hkv != 0 or
 * negative sizes, EUNSUPPORTED for head_dim other than 64/128.
 */
tilemix_status tilemix_decode_workspace_size(const tilemix_fwd_params* params, int64_t* bytes);

/*
 * tilemix_decode_fwd - the same routed attention as tilemix_prefill_fwd (identical definition of
 * s_ij, legality, route lookup, O and LSE) for a few new query tokens per sequence against a long
 * INT8 K/V cache: the decode use of the INT8 cache interface (Section 4, "cache interface";
 * Section 4.3 routed scores). With max_seqlen_q <= 8 every query of a sequence reads route row
 * cu_mtiles[b] (route_block_m >= 32).
 *
 * q8 / q_scale may both be NULL, as for tilemix_prefill_fwd: each chunk workgroup then
 * quantizes its query rows itself, bit-identically to tilemix_quantize_qk.
 * Requirements beyond tilemix_prefill_fwd: kv_int8 = 1 (k, v NULL; k8, k_scale, v8, v_scale
 * set), max_seqlen_q <= 8 and (hq / hkv) * max_seqlen_q <= 16 (EUNSUPPORTED otherwise),
 * debug_s32 NULL (EINVAL), and a workspace of tilemix_decode_workspace_size() bytes,
 * 256-byte aligned, owned by the caller (its contents on entry are irrelevant; calls that share
 * it must not overlap in time). Scores and the softmax state are fp32; P.V takes
 * fp16(P_j * v_scale[j]) against the exact fp16 of v8_j with fp32 accumulation (as the prefill
 * path rounds P to fp16).
 *
 * Implementation: a split-key pass (1024 keys of one sequence and KV head per workgroup, every
 * query row of that KV head's GQA group, scores and P.V on the matrix cores) writes per-chunk
 * max / sum / unnormalised output into the workspace; a merge pass combines them into O and LSE.
 * Both are enqueued on `stream`; the result is bitwise deterministic.
 */
tilemix_status tilemix_decode_fwd(const tilemix_fwd_params* params, void* stream);

/*
 * tilemix_decode_fwd_noalloc - tilemix_decode_fwd for callers that cannot allocate device memory
 * or pass a workspace: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. Same definition, validation, kernels and results (bitwise) as tilemix_decode_fwd;
 * the per-chunk partials live in a scratch array the library keeps on each GPU for the life of
 * the process (tilemix_decode_noalloc_max_bytes() bytes), so params->workspace and
 * params->workspace_bytes are ignored. The call allocates and frees nothing; on its first call on
 * a device it looks up that device's scratch address. Every call on one GPU shares that GPU's
 * scratch: calls that overlap in time on one GPU (other streams, other host threads) race.
 * Nothing in the scratch needs clearing: each call writes every partial it reads.
 * Errors: those of tilemix_decode_fwd, except the workspace checks; EINVAL when
 * tilemix_decode_workspace_size() of these parameters exceeds the scratch size.
 */
tilemix_status tilemix_decode_fwd_noalloc(const tilemix_fwd_params* params, void* stream);

/* Bytes of the per-device scratch of tilemix_decode_fwd_noalloc (32 MiB). */
int64_t tilemix_decode_noalloc_max_bytes(void);

/*
 * Routing policies on the device, fused with packing. The pages let the caller supply the routing
 * map R from any static or adaptive policy (Section 4.2, "Policy definition"; Limitations); these
 * calls compute R for one of two policies and write it straight into route words of the layout
 * tilemix_pack_route_mask produces ([hkv, total_mtiles, words_per_row], group g_j in word
 * g_j >> 6 at bit g_j & 63), ready for tilemix_prefill_fwd / tilemix_decode_fwd with the same
 * route geometry. For sequence b, T_b = ceil(L_k,b / (route_block_n * route_group)) groups exist;
 * bits at or past T_b are 0.
 *
 * fp16_per_mille sets the FP16 budget (the INT8 coverage is its complement):
 *   - top-k max|K| (tilemix_route_topk_maxabs): per sequence b and KV head h_k, the
 *     ceil(T_b * fp16_per_mille / 1000) groups with the largest max|K| over their keys and
 *     channels take the FP16 path (bit 0) in every route row of b (cu_mtiles[b] ..
 *     cu_mtiles[b+1]); ties go to the lower group index; the other groups below T_b are INT8
 *     (bit 1). |K| is the fp16 value, or with kv_int8 the fp32 product k_scale * |k8|. Inputs
 *     must be finite. A deterministic, data-dependent policy: the 32k GQA setting's
 *     "largest max|K| groups in FP16".
 *   - coverage-budget Bernoulli (tilemix_route_bernoulli): bit (h_k, route row r, g_j < T_b) is 0
 *     (FP16) iff x < floor(fp16_per_mille * 2^32 / 1000), x the first output word of
 *     Philox4x32-10 (Salmon et al., SC 2011) at counter (g_j, r, h_k, 0) and key (seed & 0xffffffff,
 *     seed >> 32); a data-free layout, reproducible from the seed.
 */
typedef struct tilemix_route_params {
  uint32_t struct_size;         /* sizeof(tilemix_route_params) */
  int32_t batch;                /* sequences, 1 .. 65535 */
  int32_t hkv;                  /* KV heads (route rows are per KV head), 1 .. 65535 */
  int32_t head_dim;             /* 64 or 128 (top-k only) */
  int32_t max_seqlen_k;         /* >= every L_k,b */
  const int32_t* cu_seqlens_k;  /* device [batch+1], prefix sums of L_k,b */
  const int32_t* cu_mtiles;     /* device [batch+1], prefix sums of route rows per sequence */
  int32_t total_mtiles;         /* cu_mtiles[batch] */
  int32_t route_block_n;        /* BN_r, positive multiple of 64 */
  int32_t route_group;          /* g >= 1 */
  int32_t fp16_per_mille;       /* FP16 budget, 0 .. 1000 */

  /* top-k only: the keys, fp16 [total_k, hkv, d] (strided, multiples of 8 elements, 16-byte
   * aligned) with k8 / k_scale NULL, or (kv_int8 = 1) the INT8 cache k8 [total_k, hkv, d]
   * (16-byte aligned) with k_scale [hkv, total_k] and k NULL. */
  const void* k;
  int64_t k_stride_tok, k_stride_head;
  const int8_t* k8;
  const float* k_scale;
  int64_t total_k;
  int32_t kv_int8;

  uint64_t seed;                /* Bernoulli only */

  uint64_t* route_words;        /* output [hkv, total_mtiles, words_per_row], 8-byte aligned */
  int32_t words_per_row;        /* >= ceil(ceil(max_seqlen_k / (BN_r * g)) / 64) */

  /* top-k only: device scratch of tilemix_route_workspace_size() bytes, 256-byte aligned,
   * caller-owned (per-group maxima); calls sharing it must not overlap in time. */
  void* workspace;
  int64_t workspace_bytes;
} tilemix_route_params;

/*
 * tilemix_route_workspace_size - bytes of workspace tilemix_route_topk_maxabs needs (batch, hkv,
 * max_seqlen_k, route_block_n and route_group are read): 4 * batch * hkv * ceil(max_seqlen_k /
 * (BN_r * g)), rounded up to 256. Errors: EINVAL for NULL arguments or out-of-range sizes.
 */
tilemix_status tilemix_route_workspace_size(const tilemix_route_params* params, int64_t* bytes);

/*
 * tilemix_route_topk_maxabs - the top-k max|K| policy above. A group-maximum pass (one workgroup
 * per (group, KV head, sequence), reading every key once) fills the workspace; a select-and-pack
 * pass (one workgroup per (KV head, sequence)) ranks the groups and writes the words of every
 * route row. Both are enqueued on `stream`; the result is bitwise deterministic.
 * Errors: EINVAL for a NULL or misaligned pointer, struct_size mismatch, bad strides, a budget
 * outside 0..1000, route_block_n / route_group / words_per_row out of range, a missing or small
 * workspace, k and k8 both or neither set; EUNSUPPORTED for head_dim other than 64/128 or more
 * than 8192 groups per sequence.
 */
tilemix_status tilemix_route_topk_maxabs(const tilemix_route_params* params, void* stream);

/*
 * tilemix_route_bernoulli - the coverage-budget Bernoulli policy above (k, k8, k_scale, head_dim
 * and the workspace are not read). One wavefront per route word, one lane per group. Errors:
 * EINVAL as for the top-k call where the fields apply.
 */
tilemix_status tilemix_route_bernoulli(const tilemix_route_params* params, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TILEMIX_H */
