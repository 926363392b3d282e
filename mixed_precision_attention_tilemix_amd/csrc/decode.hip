// Routed attention of a few query tokens against a long INT8 K/V cache (TileMix paper, Section 4:
// the INT8 cache interface serves decode; Section 4.3 routed-score equation; Section 3.1
// softmax), for gfx950.
//
//   decode_chunk_kernel  one workgroup per (chunk of kDecodeChunk keys, KV head, sequence) and all
//                        query rows r = i * G + g of that KV head (G query heads of the GQA group,
//                        L_q <= 8 query tokens, at most 16 rows). Each wavefront streams its own
//                        32-key tiles through the matrix cores with the rows padded to 32: the
//                        INT8 route scores with 32x32x32 int8 MFMAs of k8 against q8 (exact
//                        int32), the FP16 route with 32x32x16 fp16 MFMAs of the exact fp16 key
//                        codes against the fp16 query (fp32 accumulation); an online softmax per
//                        row in registers; and P.V as 32x32x16 fp16 MFMAs of V^T, read from the
//                        wavefront's LDS copy of the V8 tile with transposing reads and converted
//                        exactly to fp16, against fp16(P * v_scale). It writes per row the chunk's
//                        max m (log2 units), its sum l and its unnormalised O into the workspace.
//   decode_merge_kernel  one workgroup per (row, 32-channel slice, KV head, sequence): combines
//                        the chunks,
//                        O = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c with M = max_c m_c,
//                        and writes O and the natural-log LSE.
//
// Route bits come from the same packed words as the prefill path; a decode step has L_q <= 8 query
// tokens, fewer than a route tile's rows, so every row of a sequence reads route row
// cu_mtiles[b], and the 32 keys of a tile lie in one key tile: the INT8 / FP16 choice is uniform
// per wavefront.
#include <mutex>

#include "device_types.h"
#include "launch.h"

namespace tilemix {

// Scratch of the allocation-free decode entry point: the per-chunk (max, sum, O) partials of a
// call, in the layout of the caller workspace of tilemix_decode_fwd. Every GPU the library runs on
// holds its own copy until the process ends; calls on one GPU share it (and race if they overlap).
// Host code never passes this name to a kernel: on the host it is a stand-in, not a device
// address; decode_scratch() returns the address of the current device's copy.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {  // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = static_cast<float*>(addr[dev]);
  return hipSuccess;
}

namespace {

constexpr int CH = kDecodeChunk;      // keys per chunk workgroup
constexpr int MAXR = kDecodeMaxRows;  // query rows per (sequence, KV head)
constexpr int NWV = 4;                // wavefronts per chunk workgroup
constexpr int TK = 32;                // keys per tile: the key side of one 32x32 score tile
constexpr int NT = CH / (NWV * TK);   // tiles per wavefront
static_assert(NT * NWV * TK == CH, "a chunk is a whole number of tiles per wavefront");
static_assert(MAXR <= 32, "the query rows fit the 32-column side of the score tile");

typedef const __attribute__((address_space(4))) uint64_t const_u64;
typedef const __attribute__((address_space(4))) int32_t const_i32;

// Sequence offsets and route words are uniform per workgroup: scalar loads.
__device__ __forceinline__ int ld_uniform(const int32_t* p, int i) { return ((const const_i32*)p)[i]; }

// Wave-wide max (or sum) by DPP steps (within quads, 8 and 16 lanes, then row broadcasts that
// leave the total in lane 63), read back as a uniform value. Lanes a DPP step does not write
// keep the identity of the operation.
template <bool MAX, int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_step(float v) {
  const int ident = __builtin_bit_cast(int, MAX ? -INFINITY : 0.0f);
  const float u = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(ident, __builtin_bit_cast(int, v), CTRL,
                                                                        ROW_MASK, 0xF, false));
  return MAX ? fmaxf(v, u) : v + u;
}

template <bool MAX>
__device__ __forceinline__ float wave_reduce(float v) {
  v = dpp_step<MAX, 0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_step<MAX, 0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_step<MAX, 0x141, 0xF>(v);  // row_half_mirror: 8-lane groups
  v = dpp_step<MAX, 0x140, 0xF>(v);  // row_mirror: 16-lane rows
  v = dpp_step<MAX, 0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_step<MAX, 0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float wave_max(float v) { return wave_reduce<true>(v); }

// The key row a lane feeds to the score MFMA: lane n of a 32-lane half supplies M-row n, and
// with the rows permuted so (bits 2 and 3 of n swapped), score t of lane (row, half hl) belongs to
// key 16 (t >> 3) + 8 hl + (t & 7) of the tile, the layout the P.V MFMA takes P in.
__device__ __forceinline__ int perm32(int r) { return (r & 0x13) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Eight signed bytes to fp16, exactly, by the magic-number (exponent-bias) conversion: each
// byte + 128 becomes the low byte of the fp16 number 1024 + (byte + 128) (high byte 0x64, whose
// mantissa unit is 1, by a byte permute), and 1152 is subtracted.
__device__ __forceinline__ half8v i8x8_to_f16(int2v v) {
  half8v r;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t x = static_cast<uint32_t>(v[w]) ^ 0x80808080u;
    const half2v bias = {static_cast<_Float16>(1152.0f), static_cast<_Float16>(1152.0f)};
    const half2v lo = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u)) - bias;
    const half2v hi = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u)) - bias;
    r[4 * w] = lo[0];
    r[4 * w + 1] = lo[1];
    r[4 * w + 2] = hi[0];
    r[4 * w + 3] = hi[1];
  }
  return r;
}

typedef __attribute__((address_space(3))) int2v lds_int2v;

// The global loads of one 32-key tile: this lane's key row (perm32) as the INT8 score operand,
// 16 bytes per 32-byte k-step, its share of the V8 rows (16-byte chunks), and one per-key scale
// (lanes 0-31: k_scale of key jt + lane, lanes 32-63: v_scale of key jt + lane - 32), for the
// cached keys jt .. jt + 31 clamped to the last key (their scores are masked).
template <int D>
__device__ __forceinline__ void load_tile(const FwdArgs& a, int64_t k_begin, int Lk, int jt, int hk, int kr,
                                          int hl, int lane, int4v (&kf)[D / 32], int4v (&vr)[TK * D / 16 / 64],
                                          float& sc) {
  const int8_t* krow = a.k8 + ((k_begin + min(jt + kr, Lk - 1)) * a.hkv + hk) * D;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) kf[ks] = *reinterpret_cast<const int4v*>(krow + 32 * ks + 16 * hl);
  constexpr int C16 = D / 16;
#pragma unroll
  for (int u = 0; u < TK * C16 / 64; ++u) {
    const int c = lane + 64 * u;
    const int key = min(jt + c / C16, Lk - 1);
    vr[u] = *reinterpret_cast<const int4v*>(a.v8 + ((k_begin + key) * a.hkv + hk) * D + 16 * (c % C16));
  }
  const float* scales = hl ? a.v_scale : a.k_scale;
  sc = scales[static_cast<int64_t>(hk) * a.total_k + k_begin + min(jt + (lane & 31), Lk - 1)];
}

// One workgroup = one chunk of CH keys of one (sequence, KV head); each wavefront streams its own
// NT tiles of TK keys with an online softmax per query row (the next tile's key and value rows are
// loaded while the current one is computed), and the wavefronts' states are combined at the end.
template <int D>
__global__ __launch_bounds__(NWV * 64, 2) void decode_chunk_kernel(const DecodeArgs da) {
  const FwdArgs& a = da.f;
  constexpr int C16 = D / 16;          // 16-byte chunks of an int8 row
  constexpr int KS = D / 32;           // k-steps of the INT8 score MFMA
  constexpr int VR = D + 16;           // bytes per LDS row of a V8 tile (padded: no bank conflicts)
  constexpr int VU = TK * C16 / 64;    // 16-byte V8 chunks per lane per tile
  __shared__ int4v q8s[MAXR][C16];                             // int8 query rows
  __shared__ __attribute__((aligned(16))) _Float16 qh[MAXR][D];  // fp16 query rows (FP16 route)
  __shared__ float cq[MAXR];                                   // q_scale * softmax_scale * log2(e)
  __shared__ __attribute__((aligned(16))) int8_t vt8[NWV][TK * VR];  // per wavefront: V8 tile
  __shared__ __attribute__((aligned(16))) float tsc[NWV][2 * TK];    // per wavefront: k_scale, v_scale
  __shared__ float wm[NWV][MAXR], wl[NWV][MAXR];               // per wavefront: max and sum per row
  __shared__ float opart[NWV][MAXR][D];                        // per wavefront: P.V sums

  const int chunk = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.hq / a.hkv;
  const int q_begin = ld_uniform(a.cu_q, b);
  const int Lq = ld_uniform(a.cu_q, b + 1) - q_begin;
  const int64_t k_begin = ld_uniform(a.cu_k, b);
  const int Lk = ld_uniform(a.cu_k, b + 1) - static_cast<int>(k_begin);
  const int R = G * Lq;
  const int j0 = chunk * CH;
  float* part = da.part + ((static_cast<int64_t>(b) * a.hkv + hk) * da.nchunk + chunk) * da.rmax * (D + 4);
  if (R == 0) return;
  if (j0 >= Lk) {  // a sequence shorter than the longest one: an empty chunk
    for (int x = tid; x < R * (D + 4); x += NWV * 64) part[x] = (x % (D + 4) == 0) ? -INFINITY : 0.0f;
    return;
  }
  const int off = Lk - Lq;  // bottom-right causal alignment

  // The first tile's key and value rows do not depend on the queries: their loads go out first,
  // so that their latency overlaps the query rows' loads and quantization below. (The loads are
  // issued unconditionally, their keys clamped to the sequence, so every path through the loop
  // has the same loads in flight and each wait covers only older ones.)
  const int r32 = lane & 31, hl = lane >> 5;  // this lane: query row r32 of the padded 32, key half hl
  const int kr = perm32(r32);
  const int jw0 = j0 + NT * TK * w;  // first key of this wavefront's tiles
  int4v kf[KS], vr[VU];
  float scl = 0.0f;
  load_tile<D>(a, k_begin, Lk, jw0, hk, kr, hl, lane, kf, vr, scl);

  // ---- the chunk's query rows into LDS
  const bool fused_q = a.q8 == nullptr;  // quantize the query rows here instead of reading q8
  if (!fused_q) {
    for (int x = tid; x < R * C16; x += NWV * 64) {
      const int r = x / C16, c = x % C16;
      const int64_t tok = q_begin + r / G;
      const int h = hk * G + r % G;
      q8s[r][c] = *reinterpret_cast<const int4v*>(a.q8 + (tok * a.hq + h) * D + 16 * c);
    }
  }
  for (int x = tid; x < R * (D / 8); x += NWV * 64) {
    const int r = x / (D / 8), c = x % (D / 8);
    const int64_t tok = q_begin + r / G;
    const int h = hk * G + r % G;
    *reinterpret_cast<half8v*>(&qh[r][8 * c]) =
        *reinterpret_cast<const half8v*>(a.q + tok * a.q_stride_tok + h * a.q_stride_head + 8 * c);
  }
  if (!fused_q && tid < R) {
    const int64_t tok = q_begin + tid / G;
    const int h = hk * G + tid % G;
    cq[tid] = a.q_scale[static_cast<int64_t>(h) * a.total_q + tok] * a.scale_log2;
  }
  __syncthreads();
  if (fused_q) {
    // one wavefront per row: the same fp32 operations as the quantize-once pass
    // (a = max|x|, inv = 127 / a and a / 127 correctly rounded, rint, clamp)
    constexpr int EPL = D / 64;  // channels per lane
    for (int r = w; r < R; r += NWV) {
      float xv[EPL];
      float am = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        xv[e] = static_cast<float>(qh[r][EPL * lane + e]);
        am = fmaxf(am, fabsf(xv[e]));
      }
      am = wave_max(am);
      const float inv = am > 0.0f ? 127.0f / am : 0.0f;
      uint32_t packed = 0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float c = rintf(xv[e] * inv);
        c = fminf(fmaxf(c, -127.0f), 127.0f);
        packed |= static_cast<uint32_t>(static_cast<uint8_t>(static_cast<int8_t>(c))) << (8 * e);
      }
      if (EPL == 2) reinterpret_cast<uint16_t*>(&q8s[r][0])[lane] = static_cast<uint16_t>(packed);
      else reinterpret_cast<uint8_t*>(&q8s[r][0])[lane] = static_cast<uint8_t>(packed);
      if (lane == 0) cq[r] = (am > 0.0f ? am / 127.0f : 0.0f) * a.scale_log2;
    }
    __syncthreads();
  }

  const int rr = ld_uniform(a.cu_mtiles, b);
  const const_u64* wp = (const const_u64*)(a.words) + (static_cast<int64_t>(hk) * a.total_mtiles + rr) * a.wpr;

  // this lane's query row r32 is real iff r32 < R
  const bool row_valid = r32 < R;
  const int lim = !row_valid ? -1 : (a.causal ? min(Lk - 1, r32 / G + off) : Lk - 1);
  int4v qb[KS];  // the INT8 score operand of this lane's row
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qb[ks] = row_valid ? q8s[r32][2 * ks + hl] : int4v{};
  const float cqr = row_valid ? cq[r32] : 0.0f;
  const float csr = row_valid ? a.scale_log2 : 0.0f;
  // transposing V8 reads: lane m of a 16-lane group g supplies row 8 (g >> 1) + (m >> 1), bytes
  // 16 (g & 1) + 8 (m & 1); it receives channel (lane & 31) of the 8 keys 8 hl .. 8 hl + 7
  const int vsrc = (8 * hl + ((lane & 15) >> 1)) * VR + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
  int8_t* const vt = vt8[w];

  float16v o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = float16v{};
  float m = -INFINITY, l = 0.0f;

  float* const ts = tsc[w];

  for (int t = 0; t < NT; ++t) {
    const int jt = jw0 + TK * t;  // first key of the tile (uniform)
    if (jt >= Lk) break;
    int4v kn[KS], vn[VU];
    float scn = 0.0f;
    // past the wavefront's last tile the prefetch re-reads the current one (a cache hit) rather
    // than the next wavefront's first tile
    load_tile<D>(a, k_begin, Lk, min(jt + TK, jw0 + (NT - 1) * TK), hk, kr, hl, lane, kn, vn, scn);
    ts[lane] = scl;  // this tile's k_scale / v_scale, read back below by the lanes that need them

    // scores of the tile: lane (r32, hl) gets row r32 against keys jt + 16 (e >> 3) + 8 hl + (e & 7)
    const int gj = (jt / a.bn_r) / a.group;
    const bool i8 = ((wp[gj >> 6] >> (gj & 63)) & 1u) != 0u;
    float16v sc;
    float rowf;
    if (i8) {
      int16v acc = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[ks], qb[ks], acc, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[e] = static_cast<float>(acc[e]);
      rowf = cqr;
    } else {
      // the fp16 operand wants key bytes [16 s + 8 hl, +8) per 16-byte step s; this lane holds
      // [32 ks + 16 hl, +16) and swaps the missing 8 bytes with the other half of the wave
      float16v acc = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int2v mine_lo = {kf[ks][0], kf[ks][1]}, mine_hi = {kf[ks][2], kf[ks][3]};
        const int2v send = hl ? mine_lo : mine_hi;
        const int2v recv = {__shfl_xor(send[0], 32), __shfl_xor(send[1], 32)};
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int2v kb = s2 == 0 ? (hl ? recv : mine_lo) : (hl ? mine_hi : recv);
          const int kc = 32 * ks + 16 * s2 + 8 * hl;
          const half8v qv = row_valid ? *reinterpret_cast<const half8v*>(&qh[r32][kc]) : half8v{};
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(i8x8_to_f16(kb), qv, acc, 0, 0, 0);
        }
      }
      sc = acc;
      rowf = csr;
    }
    // the per-key scales of this lane's keys (two runs of 8: jt + 8 hl and jt + 16 + 8 hl)
    asm volatile("" ::: "memory");
    float ksc[16], vsc[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k0 = 16 * (q >> 1) + 8 * hl + 4 * (q & 1);
      const float4v kv = *reinterpret_cast<const float4v*>(ts + k0);
      const float4v vv = *reinterpret_cast<const float4v*>(ts + TK + k0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ksc[4 * q + i] = kv[i];
        vsc[4 * q + i] = vv[i];
      }
    }

    // log2-unit scores with the per-key factor, legality mask, tile max of the row
    float x[16];
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = jt + 16 * (e >> 3) + 8 * hl + (e & 7);
      x[e] = key > lim ? -INFINITY : sc[e] * (rowf * ksc[e]);
      mt = fmaxf(mt, x[e]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));  // the row's other key half
    if (__any(mt > m)) {
      const float alpha = mt > m ? __builtin_amdgcn_exp2f(m - mt) : 1.0f;  // m = -inf: 0
#pragma unroll
      for (int i = 0; i < D / 32; ++i) o[i] *= alpha;
      l *= alpha;
      m = fmaxf(m, mt);
    }
    half8v ph[2];  // fp16 P * v_scale, [16-key step]
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = x[e] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[e] - m);
      l += p;
      ph[e >> 3][e & 7] = static_cast<_Float16>(p * vsc[e]);
    }

    // the V8 tile into this wavefront's LDS rows, then O^T += V^T (P v_scale)^T
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int c = lane + 64 * u;
      *reinterpret_cast<int4v*>(vt + (c / C16) * VR + 16 * (c % C16)) = vr[u];
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int2v v8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_int2v*)(vt + 16 * kk * VR + 32 * dblk + vsrc));
        o[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(i8x8_to_f16(v8), ph[kk], o[dblk], 0, 0, 0);
      }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = kn[ks];
#pragma unroll
    for (int u = 0; u < VU; ++u) vr[u] = vn[u];
    scl = scn;
  }

  // this wavefront's state into LDS: lane (r32, hl) holds channels 32 dblk + 8 g + 4 hl + e
  const float l_row = l + __shfl_xor(l, 32);
  if (row_valid) {
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) opart[w][r32][32 * dblk + 8 * g + 4 * hl + e] = o[dblk][4 * g + e];
    if (hl == 0) {
      wm[w][r32] = m;
      wl[w][r32] = l_row;
    }
  }
  __syncthreads();
  // combine the wavefronts into the chunk's m, l and O
  for (int x = tid; x < R * D; x += NWV * 64) {
    const int r = x / D, c = x % D;
    float M = wm[0][r];
#pragma unroll
    for (int i = 1; i < NWV; ++i) M = fmaxf(M, wm[i][r]);
    float ov = 0.0f;
    if (M > -INFINITY) {
#pragma unroll
      for (int i = 0; i < NWV; ++i)
        if (wm[i][r] > -INFINITY) ov += __builtin_amdgcn_exp2f(wm[i][r] - M) * opart[i][r][c];
    }
    part[r * (D + 4) + 4 + c] = ov;
  }
  if (tid < R) {
    float M = wm[0][tid];
#pragma unroll
    for (int i = 1; i < NWV; ++i) M = fmaxf(M, wm[i][tid]);
    float L = 0.0f;
    if (M > -INFINITY) {
#pragma unroll
      for (int i = 0; i < NWV; ++i)
        if (wm[i][tid] > -INFINITY) L += __builtin_amdgcn_exp2f(wm[i][tid] - M) * wl[i][tid];
    }
    part[tid * (D + 4)] = M;
    part[tid * (D + 4) + 1] = L;
  }
}

constexpr int MQ = 8;          // merge: 4-channel quads per workgroup (a 32-channel slice)
constexpr int MG = 256 / MQ;   // merge: chunk groups per workgroup

// One workgroup per (query row, 32-channel slice, KV head, sequence): the chunks' maxima give M;
// 32 chunk groups rescale and sum their chunks' (l, O) for the slice, and the groups are added.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const DecodeArgs da) {
  const FwdArgs& a = da.f;
  constexpr int NS = D / (4 * MQ);  // channel slices per row
  __shared__ float smax[4];
  __shared__ float lpart[MG];
  __shared__ float4v opart[MG][MQ];
  const int r = blockIdx.x / NS, slice = blockIdx.x % NS, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int cgrp = tid / MQ, q4 = tid % MQ;  // chunk group, quad within the slice
  const int quad = slice * MQ + q4;          // 4-channel quad of the row
  const int G = a.hq / a.hkv;
  const int q_begin = ld_uniform(a.cu_q, b);
  const int Lq = ld_uniform(a.cu_q, b + 1) - q_begin;
  const int Lk = ld_uniform(a.cu_k, b + 1) - ld_uniform(a.cu_k, b);
  if (r >= G * Lq) return;
  const int nch = (Lk + CH - 1) / CH;
  const int64_t stride = static_cast<int64_t>(da.rmax) * (D + 4);
  const float* base = da.part + (static_cast<int64_t>(b) * a.hkv + hk) * da.nchunk * stride + r * (D + 4);
  // M = max over the chunks
  float M = -INFINITY;
  for (int ch = tid; ch < nch; ch += 256) M = fmaxf(M, base[ch * stride]);
  M = wave_max(M);
  if (lane == 0) smax[tid / 64] = M;
  __syncthreads();
  M = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
  float L = 0.0f;
  float4v O = {0.0f, 0.0f, 0.0f, 0.0f};
  if (M > -INFINITY) {
#pragma unroll 4
    for (int ch = cgrp; ch < nch; ch += MG) {
      const float* pc = base + ch * stride;
      const float m = pc[0];
      const float f = m > -INFINITY ? __builtin_amdgcn_exp2f(m - M) : 0.0f;
      L += f * pc[1];
      const float4v o4 = *reinterpret_cast<const float4v*>(pc + 4 + 4 * quad);
      O += f * o4;
    }
  }
  opart[cgrp][q4] = O;
  if (q4 == 0) lpart[cgrp] = L;
  __syncthreads();
  if (cgrp != 0) return;
  float Lt = 0.0f;
  float4v Ot = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < MG; ++i) {
    Lt += lpart[i];
    Ot += opart[i][q4];
  }
  const int64_t tok = q_begin + r / G;
  const int h = hk * G + r % G;
  const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
  if (a.out_f32) {
    *reinterpret_cast<float4v*>(static_cast<float*>(a.out) + (tok * a.hq + h) * D + 4 * quad) = Ot * inv;
  } else {
    half4v o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = static_cast<_Float16>(Ot[e] * inv);
    *reinterpret_cast<half4v*>(static_cast<_Float16*>(a.out) + (tok * a.hq + h) * D + 4 * quad) = o;
  }
  if (a.lse != nullptr && quad == 0)
    a.lse[static_cast<int64_t>(h) * a.total_q + tok] = Lt > 0.0f ? (M + log2f(Lt)) * 0.69314718055994531f : -INFINITY;
}

template <int D>
hipError_t launch_t(const DecodeArgs& a, int32_t batch, hipStream_t stream) {
  if (a.rmax == 0 || batch == 0) return hipSuccess;
  if (a.nchunk > 0) {
    dim3 grid(static_cast<unsigned>(a.nchunk), static_cast<unsigned>(a.f.hkv), static_cast<unsigned>(batch));
    decode_chunk_kernel<D><<<grid, dim3(NWV * 64), 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid(static_cast<unsigned>(a.rmax * (D / (4 * MQ))), static_cast<unsigned>(a.f.hkv),
            static_cast<unsigned>(batch));
  decode_merge_kernel<D><<<grid, dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int32_t batch, int32_t head_dim, hipStream_t stream) {
  return head_dim == 128 ? launch_t<128>(a, batch, stream) : launch_t<64>(a, batch, stream);
}

}  // namespace tilemix
