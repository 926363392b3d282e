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
__global__ __launch_bounds__(256) void quantize_rows_kernel(const _Float16* __restrict__ x,
                                                            int64_t n_tok, int32_t n_head,
                                                            int64_t stride_tok, int64_t stride_head,
                                                            int8_t* __restrict__ x8,
                                                            float* __restrict__ scale) {
  constexpr int G = D / 8;            // lanes per row
  constexpr int ROWS = 256 / G;       // rows per block
  const int g = threadIdx.x % G;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * ROWS + threadIdx.x / G;
  const int64_t n_rows = n_tok * n_head;
  const bool live = row < n_rows;
  const int64_t t = live ? row / n_head : 0;
  const int h = live ? static_cast<int>(row % n_head) : 0;

  half8v v = {};
  if (live) v = *reinterpret_cast<const half8v*>(x + t * stride_tok + h * stride_head + g * 8);
  float a = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(static_cast<float>(v[e])));
#pragma unroll
  for (int sh = G / 2; sh >= 1; sh >>= 1) a = fmaxf(a, __shfl_xor(a, sh, G));
  if (!live) return;

  uint64_t packed = 0;
  float s = 0.0f;
  if (a > 0.0f) {
    const float inv = 127.0f / a;  // correctly rounded (built with -fhip-fp32-correctly-rounded-divide-sqrt)
    s = a / 127.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float c = rintf(static_cast<float>(v[e]) * inv);
      c = fminf(fmaxf(c, -127.0f), 127.0f);
      packed |= static_cast<uint64_t>(static_cast<uint8_t>(static_cast<int8_t>(c))) << (8 * e);
    }
  }
  *reinterpret_cast<uint64_t*>(x8 + row * D + g * 8) = packed;
  if (g == 0) scale[static_cast<int64_t>(h) * n_tok + t] = s;
}

hipError_t launch_quantize(const void* x, int64_t n_tok, int32_t n_head, int64_t stride_tok,
                           int64_t stride_head, int8_t* x8, float* scale, int32_t head_dim,
                           hipStream_t stream) {
  const int64_t rows = n_tok * n_head;
  if (rows == 0) return hipSuccess;
  const _Float16* xp = static_cast<const _Float16*>(x);
  if (head_dim == 128) {
    const int64_t blocks = (rows + 15) / 16;
    quantize_rows_kernel<128><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(
        xp, n_tok, n_head, stride_tok, stride_head, x8, scale);
  } else {
    const int64_t blocks = (rows + 31) / 32;
    quantize_rows_kernel<64><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(
        xp, n_tok, n_head, stride_tok, stride_head, x8, scale);
  }
  return hipGetLastError();
}

}  // namespace tilemix
