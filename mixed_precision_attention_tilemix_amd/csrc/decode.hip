// Routed attention of a few query tokens against a long INT8 K/V cache (TileMix paper, Section 4:
// the INT8 cache interface serves decode; Section 4.3 routed-score equation; Section 3.1
// softmax), for gfx950.
//
// The work is HBM-bound (each cached key and value is read once per KV head), so it runs on the
// vector ALUs with coalesced 16-byte loads rather than on the matrix cores:
//
//   decode_chunk_kernel  one workgroup per (chunk of kDecodeChunk keys, KV head, sequence) and all
//                        query rows r = i * G + g of that KV head (G query heads of the GQA group,
//                        L_q query tokens). Thread t scores key j0 + t against every row: the
//                        INT8 route with 4-way int8 dot products of q8 and k8 (exact int32), the
//                        FP16 route with fp32 products of the fp16 query and the exact integer
//                        key; then a block-wide max / exp2 / sum per row, and P.V with 8-byte V8
//                        loads (16 lanes per cached row). It writes per row the chunk's max m (log2
//                        units), its sum l and its unnormalised O into the workspace.
//   decode_merge_kernel  one workgroup per (row, KV head, sequence): combines the chunks,
//                        O = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c with M = max_c m_c,
//                        and writes O and the natural-log LSE.
//
// Route bits come from the same packed words as the prefill path; a decode step has L_q <= 8 query
// tokens, fewer than a route tile's rows, so every row of a sequence reads route row
// cu_mtiles[b], and the 64 keys of a wavefront lie in one key tile: the INT8 / FP16 choice is
// uniform per wavefront.
#include "device_types.h"
#include "launch.h"

namespace tilemix {
namespace {

constexpr int CH = kDecodeChunk;      // keys per chunk workgroup
constexpr int MAXR = kDecodeMaxRows;  // query rows per (sequence, KV head)
constexpr int NWV = 4;                // wavefronts per chunk workgroup
constexpr int SL = 64;                // keys per wavefront slice (one per lane)
constexpr int NSL = CH / (NWV * SL);  // slices per wavefront
static_assert(NSL * NWV * SL == CH, "a chunk is a whole number of slices per wavefront");

typedef const __attribute__((address_space(4))) uint64_t const_u64;
typedef const __attribute__((address_space(4))) int32_t const_i32;

// Sequence offsets and route words are uniform per workgroup: scalar loads.
__device__ __forceinline__ int ld_uniform(const int32_t* p, int i) { return ((const const_i32*)p)[i]; }

// Wave-wide max / sum by DPP steps (within quads, 8 and 16 lanes, then row broadcasts that
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
__device__ __forceinline__ float wave_sum(float v) { return wave_reduce<false>(v); }

// Signed byte e (0..3) of a 32-bit word as an exact fp32 value.
__device__ __forceinline__ float sbyte(int x, int e) {
  return static_cast<float>(static_cast<int8_t>(static_cast<uint32_t>(x) >> (8 * e)));
}

// Bytes of one cached int8 row pair (this lane's key row, 16-byte loads) and its scale.
template <int D>
__device__ __forceinline__ void load_key(const FwdArgs& a, int64_t row, int tok, int hk, int4v (&kk)[D / 16],
                                         float& ksc) {
#pragma unroll
  for (int c = 0; c < D / 16; ++c) kk[c] = *reinterpret_cast<const int4v*>(a.k8 + row * D + 16 * c);
  ksc = a.k_scale[static_cast<int64_t>(hk) * a.total_k + tok];
}

// The 8-byte V8 pieces of one slice a P.V lane needs: cached rows j, j + KL, ... (clamped to the
// last key, whose P is 0 past the end), channels 8 * cg .. 8 * cg + 7.
template <int D, int KL>
__device__ __forceinline__ void load_vrows(const FwdArgs& a, int k_begin, int Lk, int j, int hk, int cg,
                                           int2v (&v)[SL / KL]) {
#pragma unroll
  for (int t = 0; t < SL / KL; ++t) {
    const int jv = min(j + KL * t, Lk - 1);
    v[t] = *reinterpret_cast<const int2v*>(a.v8 + ((static_cast<int64_t>(k_begin) + jv) * a.hkv + hk) * D + 8 * cg);
  }
}

// One workgroup = one chunk of CH keys of one (sequence, KV head); each wavefront streams its own
// NSL slices of SL keys with an online softmax per query row (the next slice's key rows are
// loaded while the current slice is scored), and the wavefronts' states are combined at the end.
// RB bounds the query rows (G * L_q).
template <int D, int RB>
__global__ __launch_bounds__(NWV * 64) void decode_chunk_kernel(const DecodeArgs da) {
  const FwdArgs& a = da.f;
  constexpr int C16 = D / 16;  // 16-byte chunks of an int8 row
  constexpr int CG = D / 8;    // P.V: channel groups of 8 per cached row
  constexpr int KL = 64 / CG;  // P.V: cached rows a wavefront covers per step
  __shared__ int4v q8s[RB][C16];        // int8 query rows
  __shared__ float qf[RB][D];           // the same rows in fp16, widened (FP16 route)
  __shared__ float cq[RB];              // q_scale * softmax_scale * log2(e) per row
  __shared__ float pvs[NWV][SL][RB];    // per wavefront: P * v_scale of the current slice
  __shared__ float wm[NWV][RB], wl[NWV][RB];  // per wavefront: final max and sum per row
  __shared__ float opart[NWV][RB][D];   // per wavefront: P.V sums

  const int chunk = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.hq / a.hkv;
  const int q_begin = ld_uniform(a.cu_q, b);
  const int Lq = ld_uniform(a.cu_q, b + 1) - q_begin;
  const int k_begin = ld_uniform(a.cu_k, b);
  const int Lk = ld_uniform(a.cu_k, b + 1) - k_begin;
  const int R = G * Lq;
  const int j0 = chunk * CH;
  float* part = da.part + ((static_cast<int64_t>(b) * a.hkv + hk) * da.nchunk + chunk) * da.rmax * (D + 4);
  if (R == 0) return;
  if (j0 >= Lk) {  // a sequence shorter than the longest one: an empty chunk
    for (int x = tid; x < R * (D + 4); x += NWV * 64) part[x] = (x % (D + 4) == 0) ? -INFINITY : 0.0f;
    return;
  }
  const int off = Lk - Lq;  // bottom-right causal alignment

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
    const half8v hv = *reinterpret_cast<const half8v*>(a.q + tok * a.q_stride_tok + h * a.q_stride_head + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[r][8 * c + e] = static_cast<float>(hv[e]);
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
        xv[e] = qf[r][EPL * lane + e];
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
  const int cg = lane % CG, kq = lane / CG;  // P.V lane = (cached row kq, channel group cg)
  const int jw0 = j0 + NSL * SL * w;         // first key of this wavefront's slices

  float m[RB], l[RB], acc[RB][8];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.0f;
  }
  // the first slice's key rows and V rows; each slice then loads the next slice's ones
  int4v kk[C16];
  float ksc = 0.0f;
  int2v vrow[SL / KL];
  if (jw0 < Lk) {
    const int jc = min(jw0 + lane, Lk - 1);
    load_key<D>(a, (static_cast<int64_t>(k_begin) + jc) * a.hkv + hk, k_begin + jc, hk, kk, ksc);
    load_vrows<D, KL>(a, k_begin, Lk, jw0 + kq, hk, cg, vrow);
  }

  for (int sl = 0; sl < NSL; ++sl) {
    const int js = jw0 + SL * sl;  // first key of the slice (uniform)
    if (js >= Lk) break;
    const int j = js + lane;
    const int jc = min(j, Lk - 1);
    const float vsc = a.v_scale[static_cast<int64_t>(hk) * a.total_k + k_begin + jc];
    // the next slice's key rows and V rows
    int4v kn[C16];
    float ksn = 0.0f;
    int2v vn[SL / KL];
    const bool more = sl + 1 < NSL && js + SL < Lk;
    if (more) {
      const int jn = min(js + SL + lane, Lk - 1);
      load_key<D>(a, (static_cast<int64_t>(k_begin) + jn) * a.hkv + hk, k_begin + jn, hk, kn, ksn);
      load_vrows<D, KL>(a, k_begin, Lk, js + SL + kq, hk, cg, vn);
    }

    // scores (log2 units) of key j against every row, by the slice's route bit
    const int gj = (js / a.bn_r) / a.group;
    const bool i8 = ((wp[gj >> 6] >> (gj & 63)) & 1u) != 0u;
    float sc[RB];
    if (i8) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if (r < R) {
          int dot = 0;
#pragma unroll
          for (int c = 0; c < C16; ++c) {
            const int4v qv = q8s[r][c];
#pragma unroll
            for (int e = 0; e < 4; ++e) dot = __builtin_amdgcn_sdot4(qv[e], kk[c][e], dot, false);
          }
          sc[r] = static_cast<float>(dot) * (cq[r] * ksc);
        }
      }
    } else {
      float dot[RB];
#pragma unroll
      for (int r = 0; r < RB; ++r) dot[r] = 0.0f;
#pragma unroll
      for (int c = 0; c < C16; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float kf[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) kf[t] = sbyte(kk[c][e], t);
#pragma unroll
          for (int r = 0; r < RB; ++r) {
            if (r < R) {
              const float4v qv = *reinterpret_cast<const float4v*>(&qf[r][16 * c + 4 * e]);
#pragma unroll
              for (int t = 0; t < 4; ++t) dot[r] = __builtin_fmaf(qv[t], kf[t], dot[r]);
            }
          }
        }
#pragma unroll
      for (int r = 0; r < RB; ++r)
        if (r < R) sc[r] = dot[r] * (a.scale_log2 * ksc);
    }

    // online softmax over this wavefront's keys; O and l are rescaled only when the max rises
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      if (r < R) {
        const bool legal = j < Lk && (!a.causal || j <= r / G + off);
        const float s = legal ? sc[r] : -INFINITY;
        const float mn = fmaxf(m[r], wave_max(s));  // uniform
        if (mn > m[r]) {
          const float alpha = __builtin_amdgcn_exp2f(m[r] - mn);  // m = -inf: 0, and O, l are 0
          l[r] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
          m[r] = mn;
        }
        const float p = s == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s - m[r]);
        l[r] += wave_sum(p);
        pvs[w][lane][r] = p * vsc;
      }
    }
    // the slice's P is read back by other lanes of this wavefront (in-order LDS within a wave)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int t = 0; t < SL / KL; ++t) {
      const int2v v8 = vrow[t];
      float vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[e] = sbyte(v8[0], e);
        vf[4 + e] = sbyte(v8[1], e);
      }
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if (r < R) {
          const float p = pvs[w][kq + KL * t][r];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r][e] = __builtin_fmaf(p, vf[e], acc[r][e]);
        }
      }
    }
    asm volatile("" ::: "memory");
    if (more) {
#pragma unroll
      for (int c = 0; c < C16; ++c) kk[c] = kn[c];
#pragma unroll
      for (int t = 0; t < SL / KL; ++t) vrow[t] = vn[t];
      ksc = ksn;
    }
  }

  // this wavefront's state: sums over the cached rows kq of a channel group, then into LDS
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    if (r < R) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = acc[r][e];
#pragma unroll
        for (int o = CG; o < 64; o <<= 1) v += __shfl_xor(v, o);
        if (kq == 0) opart[w][r][8 * cg + e] = v;
      }
      if (lane == 0) {
        wm[w][r] = m[r];
        wl[w][r] = l[r];
      }
    }
  }
  __syncthreads();
  // combine the wavefronts into the chunk's m, l and O
  for (int x = tid; x < R * D; x += NWV * 64) {
    const int r = x / D, c = x % D;
    float M = wm[0][r];
#pragma unroll
    for (int i = 1; i < NWV; ++i) M = fmaxf(M, wm[i][r]);
    float o = 0.0f;
    if (M > -INFINITY) {
#pragma unroll
      for (int i = 0; i < NWV; ++i)
        if (wm[i][r] > -INFINITY) o += __builtin_amdgcn_exp2f(wm[i][r] - M) * opart[i][r][c];
    }
    part[r * (D + 4) + 4 + c] = o;
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

constexpr int MG = 8;  // merge: chunk groups per workgroup

template <int D>
__global__ __launch_bounds__(MG * D / 4) void decode_merge_kernel(const DecodeArgs da) {
  const FwdArgs& a = da.f;
  constexpr int NT = MG * D / 4;
  __shared__ float smax[NT / 64];
  __shared__ float lpart[MG];
  __shared__ float4v opart[MG][D / 4];
  const int r = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int cgrp = tid / (D / 4), quad = tid % (D / 4);  // chunk group, 4-channel quad
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
  for (int ch = tid; ch < nch; ch += NT) M = fmaxf(M, base[ch * stride]);
  M = wave_max(M);
  if (lane == 0) smax[tid / 64] = M;
  __syncthreads();
  M = smax[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) M = fmaxf(M, smax[i]);
  // each chunk group rescales and sums its chunks, then the groups are added
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
  opart[cgrp][quad] = O;
  if (quad == 0) lpart[cgrp] = L;
  __syncthreads();
  if (cgrp != 0) return;
  float Lt = 0.0f;
  float4v Ot = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < MG; ++i) {
    Lt += lpart[i];
    Ot += opart[i][quad];
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
    if (a.rmax <= 4)
      decode_chunk_kernel<D, 4><<<grid, dim3(NWV * 64), 0, stream>>>(a);
    else if (a.rmax <= 8)
      decode_chunk_kernel<D, 8><<<grid, dim3(NWV * 64), 0, stream>>>(a);
    else
      decode_chunk_kernel<D, MAXR><<<grid, dim3(NWV * 64), 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid(static_cast<unsigned>(a.rmax), static_cast<unsigned>(a.f.hkv), static_cast<unsigned>(batch));
  decode_merge_kernel<D><<<grid, dim3(MG * D / 4), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int32_t batch, int32_t head_dim, hipStream_t stream) {
  return head_dim == 128 ? launch_t<128>(a, batch, stream) : launch_t<64>(a, batch, stream);
}

}  // namespace tilemix
