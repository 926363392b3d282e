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

constexpr int CH = kDecodeChunk;     // keys per chunk = threads per chunk workgroup
constexpr int MAXR = kDecodeMaxRows;  // query rows per (sequence, KV head)
constexpr int NWV = CH / 64;         // wavefronts per chunk workgroup

typedef const __attribute__((address_space(4))) uint64_t const_u64;
typedef const __attribute__((address_space(4))) int32_t const_i32;

// Sequence offsets and route words are uniform per workgroup: scalar loads.
__device__ __forceinline__ int ld_uniform(const int32_t* p, int i) { return ((const const_i32*)p)[i]; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Signed byte e (0..3) of a 32-bit word as an exact fp32 value.
__device__ __forceinline__ float sbyte(int x, int e) {
  return static_cast<float>(static_cast<int8_t>(static_cast<uint32_t>(x) >> (8 * e)));
}

template <int D>
__global__ __launch_bounds__(CH) void decode_chunk_kernel(const DecodeArgs da) {
  const FwdArgs& a = da.f;
  constexpr int C16 = D / 16;  // 16-byte chunks of an int8 row
  constexpr int CG = D / 8;    // P.V: channel groups of 8 per cached row
  constexpr int KL = 64 / CG;  // P.V: cached rows a wavefront covers per step
  __shared__ int4v q8s[MAXR][C16];        // int8 query rows
  __shared__ float qf[MAXR][D];           // the same rows in fp16, widened (FP16 route)
  __shared__ float cq[MAXR];              // q_scale * softmax_scale * log2(e) per row
  __shared__ float pvs[CH][MAXR];         // P * v_scale per key of the chunk and row
  __shared__ float red[NWV][MAXR];        // cross-wave reductions
  __shared__ float rowmax[MAXR];
  __shared__ float opart[NWV][MAXR][D];   // per-wave P.V sums

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
  float* part = da.part + ((static_cast<int64_t>(b) * a.hkv + hk) * da.nchunk + chunk) * da.rmax * (D + 2);
  if (R == 0) return;
  if (j0 >= Lk) {  // a sequence shorter than the longest one: an empty chunk
    for (int x = tid; x < R * (D + 2); x += CH) part[x] = (x % (D + 2) == 0) ? -INFINITY : 0.0f;
    return;
  }
  const int off = Lk - Lq;  // bottom-right causal alignment

  // ---- the chunk's query rows into LDS
  for (int x = tid; x < R * C16; x += CH) {
    const int r = x / C16, c = x % C16;
    const int64_t tok = q_begin + r / G;
    const int h = hk * G + r % G;
    q8s[r][c] = *reinterpret_cast<const int4v*>(a.q8 + (tok * a.hq + h) * D + 16 * c);
  }
  for (int x = tid; x < R * (D / 8); x += CH) {
    const int r = x / (D / 8), c = x % (D / 8);
    const int64_t tok = q_begin + r / G;
    const int h = hk * G + r % G;
    const half8v hv = *reinterpret_cast<const half8v*>(a.q + tok * a.q_stride_tok + h * a.q_stride_head + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[r][8 * c + e] = static_cast<float>(hv[e]);
  }
  if (tid < R) {
    const int64_t tok = q_begin + tid / G;
    const int h = hk * G + tid % G;
    cq[tid] = a.q_scale[static_cast<int64_t>(h) * a.total_q + tok] * a.scale_log2;
  }
  __syncthreads();

  // ---- scores of key j = j0 + tid (log2 units); keys past the end repeat the last one, masked
  const int j = j0 + tid;
  const int jc = min(j, Lk - 1);
  const int64_t krow = (static_cast<int64_t>(k_begin) + jc) * a.hkv + hk;
  int4v kk[C16];
#pragma unroll
  for (int c = 0; c < C16; ++c) kk[c] = *reinterpret_cast<const int4v*>(a.k8 + krow * D + 16 * c);
  const float ksc = a.k_scale[static_cast<int64_t>(hk) * a.total_k + k_begin + jc];
  const float vsc = a.v_scale[static_cast<int64_t>(hk) * a.total_k + k_begin + jc];
  // route bit of this wavefront's keys (one key tile), route row cu_mtiles[b]
  const int gj = (min(j0 + 64 * w, Lk - 1) / a.bn_r) / a.group;
  const int rr = ld_uniform(a.cu_mtiles, b);
  const const_u64* wp = (const const_u64*)(a.words) + (static_cast<int64_t>(hk) * a.total_mtiles + rr) * a.wpr;
  const bool i8 = ((wp[gj >> 6] >> (gj & 63)) & 1u) != 0u;

  float s[MAXR];
  if (i8) {
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      if (r < R) {
        int acc = 0;
#pragma unroll
        for (int c = 0; c < C16; ++c) {
          const int4v qv = q8s[r][c];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_sdot4(qv[e], kk[c][e], acc, false);
        }
        s[r] = static_cast<float>(acc) * (cq[r] * ksc);
      }
    }
  } else {
    float acc[MAXR];
#pragma unroll
    for (int r = 0; r < MAXR; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int c = 0; c < C16; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float kf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) kf[t] = sbyte(kk[c][e], t);
#pragma unroll
        for (int r = 0; r < MAXR; ++r) {
          if (r < R) {
            const float4v qv = *reinterpret_cast<const float4v*>(&qf[r][16 * c + 4 * e]);
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[r] = __builtin_fmaf(qv[t], kf[t], acc[r]);
          }
        }
      }
#pragma unroll
    for (int r = 0; r < MAXR; ++r)
      if (r < R) s[r] = acc[r] * (a.scale_log2 * ksc);
  }
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    if (r < R) {
      const bool legal = j < Lk && (!a.causal || j <= r / G + off);
      if (!legal) s[r] = -INFINITY;
    }
  }

  // ---- per row: chunk max, P = exp2(s - max), chunk sum
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    if (r < R) {
      const float mx = wave_max(s[r]);
      if (lane == 0) red[w][r] = mx;
    }
  }
  __syncthreads();
  if (tid < R) {
    float mx = red[0][tid];
#pragma unroll
    for (int i = 1; i < NWV; ++i) mx = fmaxf(mx, red[i][tid]);
    rowmax[tid] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    if (r < R) {
      const float p = s[r] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s[r] - rowmax[r]);
      pvs[tid][r] = p * vsc;
      const float sum = wave_sum(p);
      if (lane == 0) red[w][r] = sum;
    }
  }
  __syncthreads();
  if (tid < R) {
    float l = 0.0f;
#pragma unroll
    for (int i = 0; i < NWV; ++i) l += red[i][tid];
    part[tid * (D + 2)] = rowmax[tid];
    part[tid * (D + 2) + 1] = l;
  }

  // ---- P.V over the wavefront's 64 keys: lane = (cached row kq, channel group cg)
  const int cg = lane % CG, kq = lane / CG;
  float acc[MAXR][8];
#pragma unroll
  for (int r = 0; r < MAXR; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.0f;
#pragma unroll 4
  for (int t = 0; t < 64 / KL; ++t) {
    const int jj = 64 * w + kq + KL * t;  // key within the chunk
    const int jv = min(j0 + jj, Lk - 1);  // past the end: P is 0, any row will do
    const int2v v8 = *reinterpret_cast<const int2v*>(
        a.v8 + ((static_cast<int64_t>(k_begin) + jv) * a.hkv + hk) * D + 8 * cg);
    float vf[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vf[e] = sbyte(v8[0], e);
      vf[4 + e] = sbyte(v8[1], e);
    }
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      if (r < R) {
        const float p = pvs[jj][r];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = __builtin_fmaf(p, vf[e], acc[r][e]);
      }
    }
  }
  // sum over the cached rows kq that share a channel group, then over the wavefronts
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    if (r < R) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = acc[r][e];
#pragma unroll
        for (int o = CG; o < 64; o <<= 1) v += __shfl_xor(v, o);
        if (kq == 0) opart[w][r][8 * cg + e] = v;
      }
    }
  }
  __syncthreads();
  for (int x = tid; x < R * D; x += CH) {
    const int r = x / D, c = x % D;
    float o = 0.0f;
#pragma unroll
    for (int i = 0; i < NWV; ++i) o += opart[i][r][c];
    part[r * (D + 2) + 2 + c] = o;
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const DecodeArgs da) {
  const FwdArgs& a = da.f;
  const int r = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int c = threadIdx.x;
  const int G = a.hq / a.hkv;
  const int q_begin = ld_uniform(a.cu_q, b);
  const int Lq = ld_uniform(a.cu_q, b + 1) - q_begin;
  const int Lk = ld_uniform(a.cu_k, b + 1) - ld_uniform(a.cu_k, b);
  if (r >= G * Lq) return;
  const int nch = (Lk + CH - 1) / CH;
  const int64_t stride = static_cast<int64_t>(da.rmax) * (D + 2);
  const float* base = da.part + (static_cast<int64_t>(b) * a.hkv + hk) * da.nchunk * stride + r * (D + 2);
  float M = -INFINITY;
  for (int ch = 0; ch < nch; ++ch) M = fmaxf(M, base[ch * stride]);
  float L = 0.0f, O = 0.0f;
  if (M > -INFINITY) {
    for (int ch = 0; ch < nch; ++ch) {
      const float m = base[ch * stride];
      if (m > -INFINITY) {
        const float f = __builtin_amdgcn_exp2f(m - M);
        L += f * base[ch * stride + 1];
        O += f * base[ch * stride + 2 + c];
      }
    }
  }
  const int64_t tok = q_begin + r / G;
  const int h = hk * G + r % G;
  const float o = L > 0.0f ? O / L : 0.0f;
  if (a.out_f32)
    static_cast<float*>(a.out)[(tok * a.hq + h) * D + c] = o;
  else
    static_cast<_Float16*>(a.out)[(tok * a.hq + h) * D + c] = static_cast<_Float16>(o);
  if (a.lse != nullptr && c == 0)
    a.lse[static_cast<int64_t>(h) * a.total_q + tok] = L > 0.0f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

template <int D>
hipError_t launch_t(const DecodeArgs& a, int32_t batch, hipStream_t stream) {
  if (a.rmax == 0 || batch == 0) return hipSuccess;
  if (a.nchunk > 0) {
    dim3 grid(static_cast<unsigned>(a.nchunk), static_cast<unsigned>(a.f.hkv), static_cast<unsigned>(batch));
    decode_chunk_kernel<D><<<grid, dim3(CH), 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid(static_cast<unsigned>(a.rmax), static_cast<unsigned>(a.f.hkv), static_cast<unsigned>(batch));
  decode_merge_kernel<D><<<grid, dim3(D), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int32_t batch, int32_t head_dim, hipStream_t stream) {
  return head_dim == 128 ? launch_t<128>(a, batch, stream) : launch_t<64>(a, batch, stream);
}

}  // namespace tilemix
