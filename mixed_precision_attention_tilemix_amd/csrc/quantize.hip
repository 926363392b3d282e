// Quantize-once pass: per-token, per-head symmetric INT8 codes and fp32 scales
// (TileMix paper, Section 4.3 "quantize-once mode"; quantizer psi of Section 3.2).
//
// HBM-bound: each row of head_dim fp16 values is read once (16-byte loads, one lane per 8
// channels), its absolute maximum is reduced across the lane group with cross-lane shuffles,
// and the codes are written as one 8-byte store per lane. The scale array is head-major.
#include "device_types.h"
#include "launch.h"

namespace tilemix {

template <int D>
__device__ __forceinline__ uint64_t quantize8(const half8v v, float inv) {
  uint64_t packed = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float c = rintf(static_cast<float>(v[e]) * inv);
    c = fminf(fmaxf(c, -127.0f), 127.0f);
    packed |= static_cast<uint64_t>(static_cast<uint8_t>(static_cast<int8_t>(c))) << (8 * e);
  }
  return packed;
}

// One workgroup per (64 consecutive tokens, head): G = D/8 lanes per row, 256/G rows per pass,
// four passes' loads in flight before any arithmetic. Token-major within a head keeps the
// workgroup's scale stores in one contiguous 256-byte run. Heads vary fastest over the
// (one-dimensional) grid, so workgroups dispatched together read and write neighbouring rows of
// the same tokens instead of one head's rows a whole token stride apart.
template <int D>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const _Float16* __restrict__ x,
                                                            int64_t n_tok, int32_t n_head,
                                                            int64_t stride_tok, int64_t stride_head,
                                                            int8_t* __restrict__ x8,
                                                            float* __restrict__ scale) {
  constexpr int G = D / 8;          // lanes per row
  constexpr int RP = 256 / G;       // rows per pass
  constexpr int U = 64 / RP;        // passes: 64 tokens per workgroup
  const int g = threadIdx.x % G;
  const int h = static_cast<int>(blockIdx.x % static_cast<uint32_t>(n_head));
  const int64_t t0 = static_cast<int64_t>(blockIdx.x / static_cast<uint32_t>(n_head)) * 64 + threadIdx.x / G;

  half8v v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t t = t0 + u * RP;
    v[u] = t < n_tok ? *reinterpret_cast<const half8v*>(x + t * stride_tok + h * stride_head + g * 8)
                     : half8v{};
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(static_cast<float>(v[u][e])));
#pragma unroll
    for (int sh = G / 2; sh >= 1; sh >>= 1) a = fmaxf(a, __shfl_xor(a, sh, G));
    const int64_t t = t0 + u * RP;
    if (t >= n_tok) continue;
    const float inv = a > 0.0f ? 127.0f / a : 0.0f;  // correctly rounded (built with -fhip-fp32-correctly-rounded-divide-sqrt)
    *reinterpret_cast<uint64_t*>(x8 + (t * n_head + h) * D + g * 8) = quantize8<D>(v[u], inv);
    if (g == 0) scale[static_cast<int64_t>(h) * n_tok + t] = a > 0.0f ? a / 127.0f : 0.0f;
  }
}

// Block-wise variant (the paper's "blockwise" quantization with per-block scales): one scale per
// block of block_rows consecutive tokens of one sequence and one head, the last block of a
// sequence possibly shorter. One workgroup per (block, head, sequence) reduces the block's
// absolute maximum, then re-reads the block (from L2) to write the codes; every row of the block
// carries the block's scale, so the attention kernels read the per-token layout unchanged.
template <int D>
__global__ __launch_bounds__(256) void quantize_blocks_kernel(const _Float16* __restrict__ x,
                                                              int64_t n_tok, int32_t n_head,
                                                              int64_t stride_tok, int64_t stride_head,
                                                              const int32_t* __restrict__ cu,
                                                              int32_t block_rows,
                                                              int8_t* __restrict__ x8,
                                                              float* __restrict__ scale) {
  constexpr int G = D / 8;  // 16-byte chunks per row
  // heads vary fastest over grid.x (neighbouring workgroups read neighbouring rows of the same tokens)
  const int h = static_cast<int>(blockIdx.x % static_cast<uint32_t>(n_head)), b = blockIdx.y;
  const int64_t s0 = cu[b];
  const int64_t L = cu[b + 1] - s0;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x / static_cast<uint32_t>(n_head)) * block_rows;
  if (r0 >= L) return;  // uniform: past this sequence's tokens
  const int64_t nch = min(static_cast<int64_t>(block_rows), L - r0) * G;
  const _Float16* xb = x + (s0 + r0) * stride_tok + h * stride_head;
  // the first CAP * 256 chunks of the block stay in registers between the two passes (blocks of
  // up to 128 rows at d = 128, 256 at d = 64); larger blocks re-read the rest from L2
  constexpr int CAP = 8;
  half8v cache[CAP];
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < CAP; ++i) {
    const int64_t c = threadIdx.x + 256 * i;
    cache[i] = c < nch ? *reinterpret_cast<const half8v*>(xb + (c / G) * stride_tok + (c % G) * 8) : half8v{};
  }
#pragma unroll
  for (int i = 0; i < CAP; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(static_cast<float>(cache[i][e])));
  for (int64_t c = threadIdx.x + 256 * CAP; c < nch; c += 256) {
    const half8v v = *reinterpret_cast<const half8v*>(xb + (c / G) * stride_tok + (c % G) * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(static_cast<float>(v[e])));
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) a = fmaxf(a, __shfl_xor(a, sh));
  __shared__ float wm[4];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));

  const float inv = a > 0.0f ? 127.0f / a : 0.0f;  // correctly rounded, as in the per-token pass
  const float s = a > 0.0f ? a / 127.0f : 0.0f;
#pragma unroll
  for (int i = 0; i < CAP; ++i) {
    const int64_t c = threadIdx.x + 256 * i;
    if (c < nch) {
      const int64_t t = s0 + r0 + c / G;
      const int g = static_cast<int>(c % G);
      *reinterpret_cast<uint64_t*>(x8 + (t * n_head + h) * D + g * 8) = quantize8<D>(cache[i], inv);
      if (g == 0) scale[static_cast<int64_t>(h) * n_tok + t] = s;
    }
  }
  for (int64_t c = threadIdx.x + 256 * CAP; c < nch; c += 256) {
    const int64_t t = s0 + r0 + c / G;
    const int g = static_cast<int>(c % G);
    const half8v v = *reinterpret_cast<const half8v*>(xb + (c / G) * stride_tok + g * 8);
    *reinterpret_cast<uint64_t*>(x8 + (t * n_head + h) * D + g * 8) = quantize8<D>(v, inv);
    if (g == 0) scale[static_cast<int64_t>(h) * n_tok + t] = s;
  }
}

hipError_t launch_quantize_blocks(const void* x, int64_t n_tok, int32_t n_head, int64_t stride_tok,
                                  int64_t stride_head, const int32_t* cu, int32_t batch,
                                  int32_t max_seqlen, int32_t block_rows, int8_t* x8, float* scale,
                                  int32_t head_dim, hipStream_t stream) {
  if (n_tok == 0 || max_seqlen == 0) return hipSuccess;
  const int64_t nblk = (static_cast<int64_t>(max_seqlen) + block_rows - 1) / block_rows * n_head;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(nblk), static_cast<unsigned>(batch));
  const _Float16* xp = static_cast<const _Float16*>(x);
  if (head_dim == 128)
    quantize_blocks_kernel<128><<<grid, dim3(256), 0, stream>>>(xp, n_tok, n_head, stride_tok, stride_head,
                                                                cu, block_rows, x8, scale);
  else
    quantize_blocks_kernel<64><<<grid, dim3(256), 0, stream>>>(xp, n_tok, n_head, stride_tok, stride_head,
                                                               cu, block_rows, x8, scale);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int64_t n_tok, int32_t n_head, int64_t stride_tok,
                           int64_t stride_head, int8_t* x8, float* scale, int32_t head_dim,
                           hipStream_t stream) {
  if (n_tok == 0 || n_head == 0) return hipSuccess;
  const _Float16* xp = static_cast<const _Float16*>(x);
  const int64_t nblk = (n_tok + 63) / 64 * n_head;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(nblk));
  if (head_dim == 128)
    quantize_rows_kernel<128><<<grid, dim3(256), 0, stream>>>(xp, n_tok, n_head, stride_tok, stride_head, x8, scale);
  else
    quantize_rows_kernel<64><<<grid, dim3(256), 0, stream>>>(xp, n_tok, n_head, stride_tok, stride_head, x8, scale);
  return hipGetLastError();
}

}  // namespace tilemix
