// Fused tile-group precision-routed prefill attention for gfx950 (TileMix paper, Sections 4.1
// and 4.3): for each query tile the kernel streams key/value tiles, decodes one route bit per
// key-tile group from the packed word of its (KV head, query-tile row) (Section 4.2 lookup
// equation), computes the score tile with the FP16 or the INT8 matrix-core path, and feeds both
// into one fp32 online-softmax state (Section 3.1 recurrence) before an FP16 P.V.
//
// Work decomposition and data flow
//   * one workgroup = 8 wavefronts (two per SIMD) = 256 query rows of one query head of one
//     sequence; grid = (query heads, query tiles in reverse order, sequences). Heads vary
//     fastest and are ordered so that consecutive workgroups (which the hardware deals out to
//     the 8 XCDs in turn) keep the query heads of one KV head on one XCD and its L2, and the
//     heaviest causal tiles start first.
//   * each wavefront owns 32 query rows and computes TRANSPOSED score tiles S^T = K Q^T with
//     32x32 MFMAs, so the accumulator lands in the B-operand layout of O^T += V^T P^T: lane l
//     holds query l%32. Key rows inside each 32-key block are loaded in a permuted order (bits 2
//     and 3 of the row index swapped) so that accumulator slots t = 0..7 and 8..15 of lane l
//     hold 8 CONSECUTIVE keys each: key = 32*kb + 16*(t>>3) + 8*(l>>5) + (t&7). Row max and row
//     sum need one cross-lane exchange (lane l with lane l^32).
//   * V^T comes from a pre-pass (vt_pack.hip) that stores every 64-key tile of V transposed and
//     already swizzled, so the tile is one contiguous block and each P.V operand is a single
//     16-byte LDS read.
//   * K / K8 / k_scale / V^T tiles are double-buffered in LDS and filled with direct
//     global->LDS loads issued one tile ahead; one barrier per tile separates the buffers.
//     The fp16 Q of the workgroup stays in LDS (read only by FP16-routed tiles), the int8 Q of
//     each wavefront in registers.
//   * the route bit of a key tile is uniform over each wavefront (route tiles are multiples of
//     32 rows and 64 keys), so the FP16 / INT8 choice is a wave-uniform branch.
//   * softmax in base 2 with the score scale folded into one FMA per element; the running max
//     is only raised when a row's tile max exceeds it by more than 8 (so P < 256, exact in
//     fp32 and fp16), which makes the O rescale rare; the row sum is taken from the
//     fp16-rounded P that also feeds P.V.
#include "device_types.h"
#include "launch.h"
#include "tile_layout.h"

namespace tilemix {
namespace {

constexpr int BN = kKeyTile;  // keys per inner-loop step
constexpr int NW = 8;         // wavefronts per workgroup
constexpr int ROWS_W = 32;    // query rows per wavefront
constexpr int BM = NW * ROWS_W;
constexpr float TAU = 8.0f;   // lazy-max threshold (log2 units)

// LDS layout. Rows are unpadded; 16-byte chunks are XOR-swizzled per row so that each 1 KiB
// block stays contiguous (one direct wave load) while the rows one operand read touches fall in
// distinct banks.
template <int D>
struct Smem {
  static constexpr int RB16 = D * 2;   // bytes per fp16 row of K / Q
  static constexpr int RB8 = D;        // bytes per int8 row of K8
  static constexpr int C16 = RB16 / 16;
  static constexpr int C8 = RB8 / 16;
  static constexpr int Q16 = 0;                 // [BM][D] fp16 Q of the workgroup
  static constexpr int STAGE0 = Q16 + BM * RB16;
  static constexpr int K16 = 0;                 // offsets inside one stage
  static constexpr int K8 = K16 + BN * RB16;
  static constexpr int DK = K8 + BN * RB8;
  static constexpr int VT = DK + BN * 4;        // [D][BN] fp16 V^T, layout of vt_pack.hip
  static constexpr int STAGE = VT + D * BN * 2;
  static constexpr int BYTES = STAGE0 + 2 * STAGE;
  // The 16 lanes served together read 16 different rows at one chunk index: XOR-ing the chunk
  // with (row / rows-per-256-bytes) puts them on 16 distinct 16-byte bank groups.
  __device__ static int f16(int r) { return (r / (256 / RB16)) & (C16 - 1); }
  __device__ static int f8(int r) { return (r / (256 / RB8)) & (C8 - 1); }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

#define ONES2 half2v{static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)}

__device__ __forceinline__ half2v pk(float a, float b) {
  return half2v{static_cast<_Float16>(a), static_cast<_Float16>(b)};  // v_cvt_pk_f16_f32 (RNE)
}

typedef __attribute__((address_space(3))) void lds_void;

// One direct global->LDS load per lane: `bytes` from src to lds_block + bytes * lane.
__device__ __forceinline__ void dma16(const void* src, char* lds_block) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_block, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, char* lds_block) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_block, 4, 0, 0);
}

// Row index inside a 32-key block that MFMA row r reads: bits 2 and 3 swapped.
__device__ __forceinline__ int perm32(int r) { return (r & 0x13) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Issue the direct loads of the key tile starting at j0 (sequence-local) into stage `buf`.
// Rows past the sequence end read the last valid row; they are masked before use.
template <int D>
__device__ __forceinline__ void stage_issue(const FwdArgs& a, char* buf, const _Float16* vt_tile,
                                            int w, int lane, int j0, int Lk, int k_begin, int hk,
                                            bool need16, bool need8, bool need_dk) {
  using L = Smem<D>;
  auto key_of = [&](int row) { return static_cast<int64_t>(k_begin + min(j0 + row, Lk - 1)); };
  constexpr int R16 = 1024 / L::RB16;  // K rows per wave load
  constexpr int R8 = 1024 / L::RB8;
  if (need16) {
#pragma unroll
    for (int blk = w; blk < BN / R16; blk += NW) {
      const int row = blk * R16 + lane / L::C16;
      const int chunk = (lane % L::C16) ^ L::f16(row);
      dma16(a.k + key_of(row) * a.k_stride_tok + hk * a.k_stride_head + chunk * 8, buf + L::K16 + blk * 1024);
    }
  }
  if (need8) {
#pragma unroll
    for (int blk = w; blk < BN / R8; blk += NW) {
      const int row = blk * R8 + lane / L::C8;
      const int chunk = (lane % L::C8) ^ L::f8(row);
      dma16(a.k8 + (key_of(row) * a.hkv + hk) * D + chunk * 16, buf + L::K8 + blk * 1024);
    }
  }
  if (need_dk && w == NW - 1)
    dma4(a.k_scale + static_cast<int64_t>(hk) * a.total_k + key_of(lane), buf + L::DK);
  const char* vsrc = reinterpret_cast<const char*>(vt_tile);
#pragma unroll
  for (int blk = w; blk < D * BN * 2 / 1024; blk += NW) dma16(vsrc + blk * 1024 + lane * 16, buf + L::VT + blk * 1024);
}

// Route bits of the workgroup's wavefronts for the key tile starting at j0: bit w = route bit of
// wave w, bit 16+w = wave w computes the tile at all (it has rows in the sequence and not all of
// them are causally masked).
__device__ __forceinline__ uint32_t tile_bits(const FwdArgs& a, const uint64_t* words_hk, int mt0,
                                              int q0, int Lq, int off, int j0) {
  const int gj = (j0 / a.bn_r) / a.group;
  uint32_t bits = 0;
#pragma unroll
  for (int wv = 0; wv < NW; ++wv) {
    const int qa = q0 + ROWS_W * wv;
    const int qlast = min(qa + ROWS_W - 1, Lq - 1);
    const bool act = qa < Lq && !(a.causal && j0 > qlast + off);
    if (act) {
      const uint64_t word = words_hk[static_cast<int64_t>(mt0 + qa / a.bm_r) * a.wpr + (gj >> 6)];
      bits |= (static_cast<uint32_t>((word >> (gj & 63)) & 1u) << wv) | (1u << (16 + wv));
    }
  }
  return bits;
}

__device__ __forceinline__ bool any_fp16(uint32_t bits) { return ((bits >> 16) & ~bits & 0xffu) != 0; }
__device__ __forceinline__ bool any_int8(uint32_t bits) { return ((bits >> 16) & bits & 0xffu) != 0; }

template <int D, bool KV8>
__global__ __launch_bounds__(NW * 64, 1) void prefill_fwd_kernel(const FwdArgs a) {
  using L = Smem<D>;
  __shared__ __attribute__((aligned(1024))) char smem[L::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hl = lane >> 5;   // half of the wave: selects 8 of the 16 keys of a k-step
  const int r32 = lane & 31;  // query row of this lane within the wave

  // XCD-friendly head order: consecutive workgroups cycle through the KV heads first
  const int x = blockIdx.x;
  const int grp = a.hq / a.hkv;
  const int h = grp * (x % a.hkv) + x / a.hkv;
  const int b = blockIdx.z;
  const int n_ct = (a.max_seqlen_q + BM - 1) / BM;
  const int c = n_ct - 1 - static_cast<int>(blockIdx.y);
  const int q_begin = a.cu_q[b];
  const int Lq = a.cu_q[b + 1] - q_begin;
  const int k_begin = a.cu_k[b];
  const int Lk = a.cu_k[b + 1] - k_begin;
  const int q0 = c * BM;
  if (q0 >= Lq) return;  // uniform over the workgroup

  const int hk = h / grp;
  const int off = Lk - Lq;  // bottom-right causal alignment
  const int q_last = min(q0 + BM, Lq) - 1;
  const int key_end = a.causal ? min(Lk, q_last + off + 1) : Lk;
  const int n_tiles = key_end > 0 ? (key_end + BN - 1) / BN : 0;

  const int qa = q0 + ROWS_W * w;  // first query row of this wave
  const int my_q = qa + r32;
  const bool row_valid = my_q < Lq;
  const uint64_t* words_hk = a.words + static_cast<int64_t>(hk) * a.total_mtiles * a.wpr;
  const int mt0 = a.cu_mtiles[b];
  char* const stage0 = smem + L::STAGE0;
  const _Float16* vt_head =
      a.vt + (static_cast<int64_t>(hk) * a.vt_tiles + key_tiles_before(a.cu_k, b)) * (D * BN);

  // ---- per-lane LDS offsets of the MFMA operands (kb / dblk / kk steps are immediates)
  const int kr = perm32(r32);  // K row this lane feeds to the MFMA
  int koff16[D / 16], qoff16[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    koff16[ks] = kr * L::RB16 + 16 * ((2 * ks + hl) ^ L::f16(kr));
    qoff16[ks] = (ROWS_W * w + r32) * L::RB16 + 16 * ((2 * ks + hl) ^ L::f16(ROWS_W * w + r32));
  }
  int koff8[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) koff8[ks] = kr * L::RB8 + 16 * ((2 * ks + hl) ^ L::f8(kr));
  int voff[BN / 16];  // V^T row r32 (+32*dblk), chunk 2*kk + hl
#pragma unroll
  for (int kk = 0; kk < BN / 16; ++kk) voff[kk] = r32 * (BN * 2) + 16 * ((2 * kk + hl) ^ vt_swizzle(r32));

  // ---- resident queries: fp16 Q of the workgroup in LDS, this wave's int8 Q in registers
  for (int ch = tid; ch < BM * L::C16; ch += NW * 64) {
    const int row = ch / L::C16, col = ch % L::C16;
    int4v val = {};
    if (q0 + row < Lq)
      val = *reinterpret_cast<const int4v*>(a.q + (q_begin + q0 + row) * a.q_stride_tok +
                                            static_cast<int64_t>(h) * a.q_stride_head + col * 8);
    *reinterpret_cast<int4v*>(smem + L::Q16 + row * L::RB16 + 16 * (col ^ L::f16(row))) = val;
  }
  int4v q8f[D / 32];
  float cq = 1e-30f;  // q_scale * softmax_scale * log2(e), floored so that 0 * -inf cannot occur
  if (row_valid) {
    const int64_t tq = q_begin + my_q;
    const int8_t* q8p = a.q8 + (tq * a.hq + h) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) q8f[ks] = *reinterpret_cast<const int4v*>(q8p + 32 * ks + 16 * hl);
    cq = fmaxf(a.q_scale[static_cast<int64_t>(h) * a.total_q + tq] * a.scale_log2, 1e-30f);
  } else {
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) q8f[ks] = int4v{};
  }

  float16v o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = float16v{};
  float m_i = -INFINITY;  // running max, log2 domain
  float l_i = 0.0f;       // running normaliser

  const int my_rr = mt0 + qa / a.bm_r;
  const bool dump_me = a.dump != nullptr && h == a.dump_head && qa < Lq && my_rr >= a.dump_m0 &&
                       my_rr < a.dump_m0 + a.dump_mcount;

  // ---- prologue: tile 0 into stage 0
  uint32_t bits_next = n_tiles > 0 ? tile_bits(a, words_hk, mt0, q0, Lq, off, 0) : 0;
  if (n_tiles > 0)
    stage_issue<D>(a, stage0, vt_head, w, lane, 0, Lk, k_begin, hk, any_fp16(bits_next),
                   any_int8(bits_next), any_int8(bits_next) || KV8);
  __syncthreads();

  for (int n = 0; n < n_tiles; ++n) {
    const int j0 = n * BN;
    const uint32_t bits = bits_next;
    const char* cur = stage0 + (n & 1) * L::STAGE;
    if (n + 1 < n_tiles) {
      bits_next = tile_bits(a, words_hk, mt0, q0, Lq, off, j0 + BN);
      stage_issue<D>(a, stage0 + ((n + 1) & 1) * L::STAGE, vt_head + (n + 1) * (D * BN), w, lane,
                     j0 + BN, Lk, k_begin, hk, any_fp16(bits_next), any_int8(bits_next),
                     any_int8(bits_next) || KV8);
    }

    if ((bits >> (16 + w)) & 1u) {
      const float* dk = reinterpret_cast<const float*>(cur + L::DK);
      float16v s[2];  // [key block], pre-softmax units
      float cs;
      if ((bits >> w) & 1u) {
        // ---- INT8 path: int32 accumulation, then per-key scale (per-query scale folded in cs)
        int16v acc[2] = {};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const int4v k0 = *reinterpret_cast<const int4v*>(cur + L::K8 + koff8[ks]);
          const int4v k1 = *reinterpret_cast<const int4v*>(cur + L::K8 + 32 * L::RB8 + koff8[ks]);
          acc[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(k0, q8f[ks], acc[0], 0, 0, 0);
          acc[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(k1, q8f[ks], acc[1], 0, 0, 0);
        }
        if (dump_me && row_valid) {
          const int64_t rbase = static_cast<int64_t>(my_rr - a.dump_m0) * a.dump_ntiles;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int t = 0; t < 16; ++t) {
              const int key = j0 + 32 * kb + 16 * (t >> 3) + 8 * hl + (t & 7);
              if (key < Lk)
                a.dump[((rbase + key / a.bn_r) * a.bm_r + my_q % a.bm_r) * a.bn_r + key % a.bn_r] = acc[kb][t];
            }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int g8 = 0; g8 < 2; ++g8) {
            const float4v d0 = *reinterpret_cast<const float4v*>(dk + 32 * kb + 16 * g8 + 8 * hl);
            const float4v d1 = *reinterpret_cast<const float4v*>(dk + 32 * kb + 16 * g8 + 8 * hl + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              s[kb][8 * g8 + e] = static_cast<float>(acc[kb][8 * g8 + e]) * d0[e];
              s[kb][8 * g8 + 4 + e] = static_cast<float>(acc[kb][8 * g8 + 4 + e]) * d1[e];
            }
          }
        cs = cq;
      } else {
        // ---- FP16 path
        float16v acc[2] = {};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const half8v qv = *reinterpret_cast<const half8v*>(smem + L::Q16 + qoff16[ks]);
          const half8v k0 = *reinterpret_cast<const half8v*>(cur + L::K16 + koff16[ks]);
          const half8v k1 = *reinterpret_cast<const half8v*>(cur + L::K16 + 32 * L::RB16 + koff16[ks]);
          acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(k0, qv, acc[0], 0, 0, 0);
          acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(k1, qv, acc[1], 0, 0, 0);
        }
        if (KV8) {
          // K of the INT8 cache enters the FP16 path as exact fp16(k8): apply its scale here
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int g8 = 0; g8 < 2; ++g8) {
              const float4v d0 = *reinterpret_cast<const float4v*>(dk + 32 * kb + 16 * g8 + 8 * hl);
              const float4v d1 = *reinterpret_cast<const float4v*>(dk + 32 * kb + 16 * g8 + 8 * hl + 4);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                s[kb][8 * g8 + e] = acc[kb][8 * g8 + e] * d0[e];
                s[kb][8 * g8 + 4 + e] = acc[kb][8 * g8 + 4 + e] * d1[e];
              }
            }
        } else {
          s[0] = acc[0];
          s[1] = acc[1];
        }
        cs = a.scale_log2;  // fp16 Q is not quantized: only the softmax scale remains
      }

      // ---- legality mask (diagonal and tail tiles only)
      if ((j0 + BN > Lk) || (a.causal && j0 + BN - 1 > qa + off)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const int key = j0 + 32 * kb + 16 * (t >> 3) + 8 * hl + (t & 7);
            const bool legal = key < Lk && (!a.causal || key <= my_q + off);
            if (!legal) s[kb][t] = -INFINITY;
          }
      }

      // ---- online softmax (Section 3.1 recurrence), base 2, lazy max
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t = 0; t < 16; t += 2) mx = fmaxf(fmaxf(mx, s[kb][t]), s[kb][t + 1]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float tile_max = mx * cs;  // cs > 0
      if (__any(tile_max > m_i + TAU)) {
        const float m_new = tile_max > m_i + TAU ? tile_max : m_i;
        const float alpha = m_new > m_i ? fast_exp2(m_i - m_new) : 1.0f;
        l_i *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) o[i] *= alpha;
        m_i = m_new;
      }
      const float m_use = m_i == -INFINITY ? 0.0f : m_i;

      // ---- P = exp2(s*c - m) in fp16, O^T += V^T P^T (16 keys per MFMA step)
      float rs = 0.0f;
#pragma unroll
      for (int kk = 0; kk < BN / 16; ++kk) {
        half8v pb;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const half2v h2 = pk(fast_exp2(fmaf(s[kk >> 1][8 * (kk & 1) + e], cs, -m_use)),
                               fast_exp2(fmaf(s[kk >> 1][8 * (kk & 1) + e + 1], cs, -m_use)));
          pb[e] = h2[0];
          pb[e + 1] = h2[1];
          rs = __builtin_amdgcn_fdot2(h2, ONES2, rs, false);
        }
#pragma unroll
        for (int dblk = 0; dblk < D / 32; ++dblk) {
          const half8v vf = *reinterpret_cast<const half8v*>(cur + L::VT + dblk * 32 * (BN * 2) + voff[kk]);
          o[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pb, o[dblk], 0, 0, 0);
        }
      }
      l_i += rs + __shfl_xor(rs, 32);
    }
    __syncthreads();  // waits for this thread's direct loads, then for everyone's
  }

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) * ln 2
  if (!row_valid) return;
  const int64_t tq = q_begin + my_q;
  const float inv_l = l_i > 0.0f ? 1.0f / l_i : 0.0f;
  if (a.out_f32) {
    float* op = static_cast<float*>(a.out) + (tq * a.hq + h) * D;
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float4v v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = o[dblk][4 * g4 + e] * inv_l;
        *reinterpret_cast<float4v*>(op + dblk * 32 + 8 * g4 + 4 * hl) = v4;
      }
  } else {
    _Float16* op = static_cast<_Float16*>(a.out) + (tq * a.hq + h) * D;
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        half4v v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = static_cast<_Float16>(o[dblk][4 * g4 + e] * inv_l);
        *reinterpret_cast<half4v*>(op + dblk * 32 + 8 * g4 + 4 * hl) = v4;
      }
  }
  if (a.lse != nullptr && hl == 0)
    a.lse[static_cast<int64_t>(h) * a.total_q + tq] =
        l_i > 0.0f ? (m_i + log2f(l_i)) * 0.69314718055994531f : -INFINITY;
}

template <int D, bool KV8>
hipError_t launch_t(const FwdArgs& a, int32_t batch, hipStream_t stream) {
  const int n_ct = (a.max_seqlen_q + BM - 1) / BM;
  if (n_ct == 0 || batch == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>(a.hq), static_cast<unsigned>(n_ct), static_cast<unsigned>(batch));
  prefill_fwd_kernel<D, KV8><<<grid, dim3(NW * 64), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const FwdArgs& a, int32_t batch, int32_t head_dim, bool kv_int8,
                          hipStream_t stream) {
  if (head_dim == 128)
    return kv_int8 ? launch_t<128, true>(a, batch, stream) : launch_t<128, false>(a, batch, stream);
  return kv_int8 ? launch_t<64, true>(a, batch, stream) : launch_t<64, false>(a, batch, stream);
}

}  // namespace tilemix
