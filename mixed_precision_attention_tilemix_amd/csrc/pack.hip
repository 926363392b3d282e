// Route-map packing: b = sum_j R_j 2^j over the key-tile groups of one (KV head, query-tile
// row), 64 groups per word (TileMix paper, Section 4.2, packing equation); rows with more than
// 64 groups continue in the following words.
#include "device_types.h"
#include "launch.h"

namespace tilemix {

__global__ __launch_bounds__(256) void pack_route_kernel(const uint8_t* __restrict__ route,
                                                         int64_t rows, int32_t t_mask,
                                                         uint64_t* __restrict__ words, int32_t wpr) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= rows * wpr) return;
  const int64_t r = idx / wpr;
  const int w = static_cast<int>(idx % wpr);
  const uint8_t* src = route + r * t_mask;
  uint64_t word = 0;
  const int g0 = 64 * w;
  const int g1 = min(t_mask, g0 + 64);
  for (int g = g0; g < g1; ++g) word |= static_cast<uint64_t>(src[g] != 0) << (g - g0);
  words[idx] = word;
}

hipError_t launch_pack(const uint8_t* route, int64_t rows, int32_t t_mask, uint64_t* words,
                       int32_t words_per_row, hipStream_t stream) {
  const int64_t n = rows * words_per_row;
  if (n == 0) return hipSuccess;
  pack_route_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream>>>(
      route, rows, t_mask, words, words_per_row);
  return hipGetLastError();
}

}  // namespace tilemix
