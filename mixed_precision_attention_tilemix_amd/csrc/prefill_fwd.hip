// Fused tile-group precision-routed prefill attention for gfx950 (TileMix paper, Sections 4.1
// and 4.3): for each query tile the kernel streams key/value tiles, decodes one route bit per
// key-tile group from the packed word of its (KV head, query-tile row) (Section 4.2 lookup
// equation), computes the score tile with the FP16 or the INT8 matrix-core path, and feeds both
// into one fp32 online-softmax state (Section 3.1 recurrence) before an FP16 P.V.
//
// Work decomposition
//   * one workgroup = NW wavefronts = 32*NW query rows of one query head of one sequence;
//     grid = (query heads, query tiles in reverse order, sequences): heads vary fastest so that
//     the heaviest causal tiles of every head start first and the query heads that share a KV
//     head run side by side.
//   * each wavefront owns 32 query rows and computes the TRANSPOSED score tile S^T = K Q^T with
//     32x32 MFMAs, so that the accumulator lands directly in the B-operand layout of the P.V
//     product O^T += V^T P^T: lane l holds query l%32 and keys 8*(t/4) + 4*(l/32) + t%4 of a
//     32-key block in accumulator slot t. Row max and row sum need one cross-lane exchange
//     (lane l with lane l^32).
//   * the V^T operand is read from the row-major V tile with the gfx950 transposing LDS read
//     (ds_read_b64_tr_b16), which hands lane i of each 16-lane group the 4 keys of channel i.
//   * the route bit of a key tile is uniform over the wavefront (route tiles are multiples of
//     32 rows and 64 keys), so the FP16 / INT8 choice is a wave-uniform branch.
#include "device_types.h"
#include "launch.h"

namespace tilemix {
namespace {

constexpr int BN = 64;  // keys per inner-loop step (one or more steps per route tile column)

template <int D, bool KV8>
struct Smem {
  static constexpr int K16_STRIDE = D * 2 + 32;  // bytes; +32 keeps 4-row groups bank-disjoint
  static constexpr int K8_STRIDE = D + 16;
  static constexpr int V16_STRIDE = D * 2 + 32;
  static constexpr int K16 = 0;
  static constexpr int K8 = K16 + BN * K16_STRIDE;
  static constexpr int DK = K8 + BN * K8_STRIDE;
  static constexpr int V16 = DK + BN * 4;
  static constexpr int DV = V16 + BN * V16_STRIDE;
  static constexpr int BYTES = DV + BN * 4;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ half8v cat8(short4v lo, short4v hi) {
  half4v a = __builtin_bit_cast(half4v, lo);
  half4v b = __builtin_bit_cast(half4v, hi);
  return half8v{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// 16 int8 values -> 16 fp16 values (exact: |x| <= 127).
__device__ __forceinline__ void int8x16_to_half(int4v src, half8v* lo, half8v* hi) {
  const int8_t* s = reinterpret_cast<const int8_t*>(&src);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    (*lo)[e] = static_cast<_Float16>(s[e]);
    (*hi)[e] = static_cast<_Float16>(s[8 + e]);
  }
}

template <int D, int NW, bool KV8>
__global__ __launch_bounds__(NW * 64) void prefill_fwd_kernel(const FwdArgs a) {
  using L = Smem<D, KV8>;
  constexpr int BM = 32 * NW;
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hl = lane >> 5;       // which half of the wave (key sub-rows of the C layout)
  const int r32 = lane & 31;      // query row within the wave / key row within a block

  const int h = blockIdx.x;
  const int b = blockIdx.z;
  const int n_ct = (a.max_seqlen_q + BM - 1) / BM;
  const int c = n_ct - 1 - static_cast<int>(blockIdx.y);
  const int q_begin = a.cu_q[b];
  const int Lq = a.cu_q[b + 1] - q_begin;
  const int k_begin = a.cu_k[b];
  const int Lk = a.cu_k[b + 1] - k_begin;
  const int q0 = c * BM;
  if (q0 >= Lq) return;  // uniform over the workgroup

  const int hk = h / (a.hq / a.hkv);
  const int off = Lk - Lq;  // bottom-right causal alignment
  const int q_last = min(q0 + BM, Lq) - 1;
  const int key_end = a.causal ? min(Lk, q_last + off + 1) : Lk;
  const int n_tiles = key_end > 0 ? (key_end + BN - 1) / BN : 0;

  const int qa = q0 + 32 * w;          // first query row of this wave
  const bool wave_active = qa < Lq;
  const int my_q = qa + r32;           // this lane's query row (local to the sequence)
  const bool row_valid = my_q < Lq;

  // ---- resident query fragments: B operands of S^T = K Q^T
  half8v qf[D / 16];
  int4v q8f[D / 32];
  float cq = 0.0f;  // q_scale * softmax_scale * log2(e)
  if (row_valid) {
    const int64_t tq = q_begin + my_q;
    const _Float16* qp = a.q + tq * a.q_stride_tok + static_cast<int64_t>(h) * a.q_stride_head;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qf[ks] = *reinterpret_cast<const half8v*>(qp + 16 * ks + 8 * hl);
    const int8_t* q8p = a.q8 + (tq * a.hq + h) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      q8f[ks] = *reinterpret_cast<const int4v*>(q8p + 32 * ks + 16 * hl);
    cq = a.q_scale[static_cast<int64_t>(h) * a.total_q + tq] * a.scale_log2;
  } else {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = half8v{};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) q8f[ks] = int4v{};
  }

  const uint64_t* words_hk = a.words + static_cast<int64_t>(hk) * a.total_mtiles * a.wpr;
  const int mt0 = a.cu_mtiles[b];
  const int my_route_row = mt0 + qa / a.bm_r;
  const bool dump_wave = a.dump != nullptr && h == a.dump_head && wave_active &&
                         my_route_row >= a.dump_m0 && my_route_row < a.dump_m0 + a.dump_mcount;

  float16v o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = float16v{};
  float m_i = -INFINITY;  // running max, log2 domain
  float l_i = 0.0f;       // running normaliser

  const int G16 = lane >> 4, s16 = lane & 15;  // transposing-read lane coordinates

  for (int n = 0; n < n_tiles; ++n) {
    const int j0 = n * BN;
    const int gj = (j0 / a.bn_r) / a.group;
    // route bits of every wave of the workgroup for this key tile
    bool need16 = false, need8 = false, my_compute = false;
    int my_bit = 0;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) {
      const int qa_w = q0 + 32 * wv;
      if (qa_w >= Lq) continue;
      const int qlast_w = min(qa_w + 31, Lq - 1);
      if (a.causal && j0 > qlast_w + off) continue;  // tile fully masked for that wave
      const int rr = mt0 + qa_w / a.bm_r;
      const uint64_t word = words_hk[static_cast<int64_t>(rr) * a.wpr + (gj >> 6)];
      const int bit = static_cast<int>((word >> (gj & 63)) & 1u);
      need8 |= bit != 0;
      need16 |= bit == 0;
      if (wv == w) {
        my_compute = true;
        my_bit = bit;
      }
    }

    __syncthreads();  // the previous tile's readers are done with LDS

    // ---- stage the key/value tile into LDS (zero rows past the sequence end)
    if (!KV8) {
      if (need16) {
        for (int ch = tid; ch < BN * (D / 8); ch += NT) {
          const int row = ch / (D / 8), col = ch % (D / 8);
          const int key = j0 + row;
          half8v val = {};
          if (key < Lk)
            val = *reinterpret_cast<const half8v*>(a.k + (k_begin + key) * a.k_stride_tok +
                                                   hk * a.k_stride_head + col * 8);
          *reinterpret_cast<half8v*>(smem + L::K16 + row * L::K16_STRIDE + col * 16) = val;
        }
      }
      if (need8) {
        for (int ch = tid; ch < BN * (D / 16); ch += NT) {
          const int row = ch / (D / 16), col = ch % (D / 16);
          const int key = j0 + row;
          int4v val = {};
          if (key < Lk)
            val = *reinterpret_cast<const int4v*>(a.k8 + ((k_begin + key) * static_cast<int64_t>(a.hkv) + hk) * D + col * 16);
          *reinterpret_cast<int4v*>(smem + L::K8 + row * L::K8_STRIDE + col * 16) = val;
        }
        for (int row = tid; row < BN; row += NT) {
          const int key = j0 + row;
          reinterpret_cast<float*>(smem + L::DK)[row] =
              key < Lk ? a.k_scale[static_cast<int64_t>(hk) * a.total_k + k_begin + key] : 0.0f;
        }
      }
      for (int ch = tid; ch < BN * (D / 8); ch += NT) {
        const int row = ch / (D / 8), col = ch % (D / 8);
        const int key = j0 + row;
        half8v val = {};
        if (key < Lk)
          val = *reinterpret_cast<const half8v*>(a.v + (k_begin + key) * a.v_stride_tok +
                                                 hk * a.v_stride_head + col * 8);
        *reinterpret_cast<half8v*>(smem + L::V16 + row * L::V16_STRIDE + col * 16) = val;
      }
    } else {
      // INT8 cache: K8 feeds the INT8 path directly and, converted exactly to fp16, the FP16
      // path; V8 is converted exactly to fp16 and its scale is applied to P.
      for (int ch = tid; ch < BN * (D / 16); ch += NT) {
        const int row = ch / (D / 16), col = ch % (D / 16);
        const int key = j0 + row;
        int4v kv = {}, vv = {};
        if (key < Lk) {
          const int64_t base = ((k_begin + key) * static_cast<int64_t>(a.hkv) + hk) * D + col * 16;
          kv = *reinterpret_cast<const int4v*>(a.k8 + base);
          vv = *reinterpret_cast<const int4v*>(a.v8 + base);
        }
        if (need8) *reinterpret_cast<int4v*>(smem + L::K8 + row * L::K8_STRIDE + col * 16) = kv;
        if (need16) {
          half8v lo, hi;
          int8x16_to_half(kv, &lo, &hi);
          *reinterpret_cast<half8v*>(smem + L::K16 + row * L::K16_STRIDE + col * 32) = lo;
          *reinterpret_cast<half8v*>(smem + L::K16 + row * L::K16_STRIDE + col * 32 + 16) = hi;
        }
        half8v lo, hi;
        int8x16_to_half(vv, &lo, &hi);
        *reinterpret_cast<half8v*>(smem + L::V16 + row * L::V16_STRIDE + col * 32) = lo;
        *reinterpret_cast<half8v*>(smem + L::V16 + row * L::V16_STRIDE + col * 32 + 16) = hi;
      }
      for (int row = tid; row < BN; row += NT) {
        const int key = j0 + row;
        const int64_t si = static_cast<int64_t>(hk) * a.total_k + k_begin + key;
        reinterpret_cast<float*>(smem + L::DK)[row] = key < Lk ? a.k_scale[si] : 0.0f;
        reinterpret_cast<float*>(smem + L::DV)[row] = key < Lk ? a.v_scale[si] : 0.0f;
      }
    }

    __syncthreads();

    if (!my_compute) continue;

    // ---- score tile S^T (64 keys x 32 queries) in the log2 domain
    float s[2][16];
    const float* dk = reinterpret_cast<const float*>(smem + L::DK);
    if (my_bit) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        int16v acc = {};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const int4v av = *reinterpret_cast<const int4v*>(
              smem + L::K8 + (blk * 32 + r32) * L::K8_STRIDE + 32 * ks + 16 * hl);
          acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, q8f[ks], acc, 0, 0, 0);
        }
        if (dump_wave && row_valid) {
          const int i_in = my_q % a.bm_r;
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const int key = j0 + blk * 32 + 8 * (t / 4) + 4 * hl + (t % 4);
            if (key < Lk) {
              const int64_t idx =
                  ((static_cast<int64_t>(my_route_row - a.dump_m0) * a.dump_ntiles + key / a.bn_r) *
                       a.bm_r + i_in) * a.bn_r + key % a.bn_r;
              a.dump[idx] = acc[t];
            }
          }
        }
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4v dk4 = *reinterpret_cast<const float4v*>(dk + blk * 32 + 8 * g4 + 4 * hl);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s[blk][4 * g4 + e] = static_cast<float>(acc[4 * g4 + e]) * dk4[e] * cq;
        }
      }
    } else {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        float16v acc = {};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const half8v av = *reinterpret_cast<const half8v*>(
              smem + L::K16 + (blk * 32 + r32) * L::K16_STRIDE + (16 * ks + 8 * hl) * 2);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, qf[ks], acc, 0, 0, 0);
        }
        if (KV8) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const float4v dk4 = *reinterpret_cast<const float4v*>(dk + blk * 32 + 8 * g4 + 4 * hl);
#pragma unroll
            for (int e = 0; e < 4; ++e) s[blk][4 * g4 + e] = acc[4 * g4 + e] * (dk4[e] * a.scale_log2);
          }
        } else {
#pragma unroll
          for (int t = 0; t < 16; ++t) s[blk][t] = acc[t] * a.scale_log2;
        }
      }
    }

    // ---- legality mask (diagonal and tail tiles only)
    const bool need_mask = (j0 + BN > Lk) || (a.causal && j0 + BN - 1 > qa + off);
    if (need_mask) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int key = j0 + blk * 32 + 8 * (t / 4) + 4 * hl + (t % 4);
          const bool legal = key < Lk && (!a.causal || key <= my_q + off);
          if (!legal) s[blk][t] = -INFINITY;
        }
    }

    // ---- online softmax update (Section 3.1 recurrence, fp32 state, base-2 exponentials)
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int t = 0; t < 16; ++t) mx = fmaxf(mx, s[blk][t]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_i, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = fast_exp2(m_i - m_use);
    float rs = 0.0f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        s[blk][t] = fast_exp2(s[blk][t] - m_use);
        rs += s[blk][t];
      }
    rs += __shfl_xor(rs, 32);
    l_i = l_i * alpha + rs;
    m_i = m_new;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) o[i] *= alpha;

    if (KV8) {
      const float* dv = reinterpret_cast<const float*>(smem + L::DV);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4v dv4 = *reinterpret_cast<const float4v*>(dv + blk * 32 + 8 * g4 + 4 * hl);
#pragma unroll
          for (int e = 0; e < 4; ++e) s[blk][4 * g4 + e] *= dv4[e];
        }
    }

    // ---- O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
    for (int kk = 0; kk < BN / 16; ++kk) {
      half8v pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = static_cast<_Float16>(s[kk / 2][8 * (kk % 2) + e]);
      const int row0 = 16 * kk + 4 * (G16 >> 1) + (s16 >> 2);
#pragma unroll
      for (int dblk = 0; dblk < D / 32; ++dblk) {
        const int col = dblk * 32 + 16 * (G16 & 1) + 4 * (s16 & 3);
        const char* p0 = smem + L::V16 + row0 * L::V16_STRIDE + col * 2;
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(p0));
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(p0 + 8 * L::V16_STRIDE));
        o[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cat8(lo, hi), pb, o[dblk], 0, 0, 0);
      }
    }
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

template <int D, int NW, bool KV8>
hipError_t launch_t(const FwdArgs& a, int32_t batch, hipStream_t stream) {
  constexpr int BM = 32 * NW;
  const int n_ct = (a.max_seqlen_q + BM - 1) / BM;
  if (n_ct == 0 || batch == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>(a.hq), static_cast<unsigned>(n_ct), static_cast<unsigned>(batch));
  prefill_fwd_kernel<D, NW, KV8><<<grid, dim3(NW * 64), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const FwdArgs& a, int32_t batch, int32_t head_dim, bool kv_int8,
                          hipStream_t stream) {
  constexpr int NW = 4;
  if (head_dim == 128)
    return kv_int8 ? launch_t<128, NW, true>(a, batch, stream) : launch_t<128, NW, false>(a, batch, stream);
  return kv_int8 ? launch_t<64, NW, true>(a, batch, stream) : launch_t<64, NW, false>(a, batch, stream);
}

}  // namespace tilemix
