// Routing policies computed on the device and written straight into packed route words (TileMix
// paper, Section 4.2: the routing map R may come from any static or adaptive policy, and is
// packed as b = sum_j R_j 2^j, 64 groups per word). Two policies:
//   * top-k by max|K|: per (sequence, KV head) the ceil(T * per_mille / 1000) key-tile groups with
//     the largest max|K| are FP16 (bit 0) in every route row of the sequence, ties to the lower
//     group index; the other groups below T are INT8 (bit 1).
//   * coverage-budget Bernoulli: bit (h_k, row, g_j) is FP16 iff the first word of
//     Philox4x32-10(counter (g_j, row, h_k, 0), key (seed_lo, seed_hi)) is below thr.
// Groups at or past a sequence's T = ceil(L_k / (BN_r * g)) are 0 in both.
#include "device_types.h"
#include "launch.h"

namespace tilemix {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ uint32_t fold_abs_f16(uint32_t m, uint32_t w) {
  // |x| of two fp16 values as bit patterns, which order like the values when non-negative
  return max(m, max(w & 0x7fffu, (w >> 16) & 0x7fffu));
}

__device__ __forceinline__ int fold_abs_i8(int m, uint32_t w) {
#pragma unroll
  for (int e = 0; e < 4; ++e) m = max(m, abs(static_cast<int>(static_cast<int8_t>(w >> (8 * e)))));
  return m;
}

// max|K| of keys [j0, j1) of one KV head, fp16 keys; this lane's share.
template <int D>
__device__ __forceinline__ float lane_max_f16(const RouteArgs& a, int h, int64_t k0, int64_t j0,
                                              int64_t j1) {
  constexpr int LPR = D / 8;              // lanes per key row, 16 bytes each
  constexpr int RPP = kThreads / LPR;     // key rows per pass of the workgroup
  constexpr int U = 8;                    // independent loads in flight per lane
  const uint16_t* base = a.k + h * a.k_stride_head + (threadIdx.x % LPR) * 8;
  uint32_t mb = 0;
  for (int64_t j = j0 + threadIdx.x / LPR; j < j1; j += static_cast<int64_t>(RPP) * U) {
    uint4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t jj = j + u * RPP;
      x[u] = jj < j1 ? *reinterpret_cast<const uint4*>(base + (k0 + jj) * a.k_stride_tok)
                     : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      mb = fold_abs_f16(mb, x[u].x);
      mb = fold_abs_f16(mb, x[u].y);
      mb = fold_abs_f16(mb, x[u].z);
      mb = fold_abs_f16(mb, x[u].w);
    }
  }
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(mb)));
}

// max over keys [j0, j1) of k_scale * max|k8| (fp32 products), INT8 cache; this lane's share.
template <int D>
__device__ __forceinline__ float lane_max_i8(const RouteArgs& a, int h, int64_t k0, int64_t j0,
                                             int64_t j1) {
  constexpr int LPR = D / 16;
  constexpr int RPP = kThreads / LPR;
  constexpr int U = 8;
  const int8_t* base = a.k8 + static_cast<int64_t>(h) * D + (threadIdx.x % LPR) * 16;
  const int64_t tok_stride = static_cast<int64_t>(a.hkv) * D;
  const float* sc = a.k_scale + static_cast<int64_t>(h) * a.total_k + k0;
  float m = 0.0f;
  for (int64_t j = j0 + threadIdx.x / LPR; j < j1; j += static_cast<int64_t>(RPP) * U) {
    uint4 x[U];
    float s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t jj = j + u * RPP;
      const bool in = jj < j1;
      x[u] = in ? *reinterpret_cast<const uint4*>(base + (k0 + jj) * tok_stride) : make_uint4(0u, 0u, 0u, 0u);
      s[u] = in ? sc[jj] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int am = fold_abs_i8(0, x[u].x);
      am = fold_abs_i8(am, x[u].y);
      am = fold_abs_i8(am, x[u].z);
      am = fold_abs_i8(am, x[u].w);
      // fl(s * a) is non-decreasing in a, so the lane maxima combine to the per-key product
      m = fmaxf(m, s[u] * static_cast<float>(am));
    }
  }
  return m;
}

// One workgroup per (group g_j, KV head, sequence): gmax[b][h][g_j] = max|K| over the group.
template <int D, bool KV8>
__global__ __launch_bounds__(kThreads) void group_maxabs_kernel(const RouteArgs a) {
  const int gj = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t k0 = a.cu_k[b];
  const int64_t Lk = a.cu_k[b + 1] - k0;
  const int64_t j0 = static_cast<int64_t>(gj) * a.span;
  if (j0 >= Lk) return;  // uniform: the group lies past this sequence's keys
  const int64_t j1 = min(Lk, j0 + a.span);
  float m = KV8 ? lane_max_i8<D>(a, h, k0, j0, j1) : lane_max_f16<D>(a, h, k0, j0, j1);
  m = wave_max(m);
  __shared__ float wm[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = wm[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, wm[i]);
    a.gmax[(static_cast<int64_t>(b) * a.hkv + h) * a.tmax + gj] = r;
  }
}

// One workgroup per (KV head, sequence): rank the T group maxima (descending, lower index first
// on ties), keep the first ceil(T * per_mille / 1000) as FP16 and write the packed words to every
// route row of the sequence.
__global__ __launch_bounds__(kThreads) void topk_pack_kernel(const RouteArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  __shared__ float s[kRouteMaxGroups];
  __shared__ unsigned long long w[kRouteMaxGroups / 64];
  const int64_t Lk = a.cu_k[b + 1] - a.cu_k[b];
  const int T = static_cast<int>(min(static_cast<int64_t>(a.tmax), (Lk + a.span - 1) / a.span));
  const int nw = (T + 63) / 64;
  const float* g = a.gmax + (static_cast<int64_t>(b) * a.hkv + h) * a.tmax;
  for (int i = threadIdx.x; i < T; i += kThreads) s[i] = g[i];
  for (int i = threadIdx.x; i < nw; i += kThreads) w[i] = 0ull;
  __syncthreads();
  const int nsel = static_cast<int>((static_cast<int64_t>(T) * a.per_mille + 999) / 1000);
  for (int i = threadIdx.x; i < T; i += kThreads) {
    bool int8 = true;
    if (nsel >= T) {
      int8 = false;
    } else if (nsel > 0) {
      const float v = s[i];
      int rank = 0;  // groups ordered before group i
      for (int j = 0; j < T; ++j) {
        const float u = s[j];
        rank += (u > v) | ((u == v) & (j < i));
      }
      int8 = rank >= nsel;
    }
    if (int8) atomicOr(&w[i >> 6], 1ull << (i & 63));
  }
  __syncthreads();
  const int64_t r0 = max(0, a.cu_mtiles[b]);
  const int64_t r1 = min(a.cu_mtiles[b + 1], a.total_mtiles);
  if (r1 <= r0) return;
  uint64_t* out = a.words + (static_cast<int64_t>(h) * a.total_mtiles + r0) * a.wpr;
  const int64_t n = (r1 - r0) * a.wpr;
  for (int64_t i = threadIdx.x; i < n; i += kThreads) {
    const int c = static_cast<int>(i % a.wpr);
    out[i] = c < nw ? w[c] : 0ull;
  }
}

// First output word of Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011): ten rounds of the
// two multiply-high/low mixes, the key advanced by the Weyl constants between rounds.
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0;
    const uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return c0;
}

// One wavefront per route word (h_k, row, word c); lane l draws group 64 c + l and a ballot
// assembles the word.
__global__ __launch_bounds__(kThreads) void bernoulli_pack_kernel(const RouteArgs a, int64_t n) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + threadIdx.x / 64;
  if (idx >= n) return;  // uniform across the wavefront
  const int lane = threadIdx.x & 63;
  const int c = static_cast<int>(idx % a.wpr);
  const int64_t hr = idx / a.wpr;
  const int r = static_cast<int>(hr % a.total_mtiles);
  const int h = static_cast<int>(hr / a.total_mtiles);
  // the sequence owning route row r: the last b with cu_mtiles[b] <= r
  int lo = 0, hi = a.batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu_mtiles[mid] <= r) lo = mid;
    else hi = mid;
  }
  const int64_t Lk = a.cu_k[lo + 1] - a.cu_k[lo];
  const int64_t T = (Lk + a.span - 1) / a.span;
  const int64_t g = static_cast<int64_t>(64) * c + lane;
  bool int8 = false;
  if (g < T) {
    const uint32_t x = philox_word0(static_cast<uint32_t>(g), static_cast<uint32_t>(r),
                                    static_cast<uint32_t>(h), 0u, a.seed_lo, a.seed_hi);
    int8 = static_cast<uint64_t>(x) >= a.thr;
  }
  const uint64_t word = __ballot(int8);
  if (lane == 0) a.words[idx] = word;
}

template <int D>
hipError_t launch_topk_d(const RouteArgs& a, bool kv_int8, hipStream_t stream) {
  if (a.tmax > 0) {
    const dim3 grid(static_cast<unsigned>(a.tmax), static_cast<unsigned>(a.hkv), static_cast<unsigned>(a.batch));
    if (kv_int8) group_maxabs_kernel<D, true><<<grid, dim3(kThreads), 0, stream>>>(a);
    else group_maxabs_kernel<D, false><<<grid, dim3(kThreads), 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  topk_pack_kernel<<<dim3(static_cast<unsigned>(a.hkv), static_cast<unsigned>(a.batch)), dim3(kThreads), 0,
                     stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_topk(const RouteArgs& a, int32_t head_dim, bool kv_int8, hipStream_t stream) {
  return head_dim == 64 ? launch_topk_d<64>(a, kv_int8, stream) : launch_topk_d<128>(a, kv_int8, stream);
}

hipError_t launch_route_bernoulli(const RouteArgs& a, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(a.hkv) * a.total_mtiles * a.wpr;
  if (n == 0) return hipSuccess;
  constexpr int64_t kWordsPerBlock = kThreads / 64;
  bernoulli_pack_kernel<<<dim3(static_cast<unsigned>((n + kWordsPerBlock - 1) / kWordsPerBlock)),
                          dim3(kThreads), 0, stream>>>(a, n);
  return hipGetLastError();
}

}  // namespace tilemix
