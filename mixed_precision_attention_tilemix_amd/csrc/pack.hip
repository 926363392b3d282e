// Route-map packing: b = sum_j R_j 2^j over the key-tile groups of one (KV head, query-tile
// row), 64 groups per word (TileMix paper, Section 4.2, packing equation); rows with more than
// 64 groups continue in the following words.
#include "device_types.h"
#include "launch.h"

namespace tilemix {

// One wavefront per output word: lane i reads group 64 w + i of the row (one coalesced byte per
// lane) and the wave's ballot of "nonzero" is the word itself (bit i = lane i).
__global__ __launch_bounds__(256) void pack_route_kernel(const uint8_t* __restrict__ route,
                                                         int64_t rows, int32_t t_mask,
                                                         uint64_t* __restrict__ words, int32_t wpr) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (idx >= rows * wpr) return;  // uniform over the wavefront
  const int lane = threadIdx.x & 63;
  const int64_t r = idx / wpr;
  const int g = 64 * static_cast<int>(idx % wpr) + lane;
  const bool bit = g < t_mask && route[r * t_mask + g] != 0;
  const uint64_t word = __ballot(bit);
  if (lane == 0) words[idx] = word;
}

hipError_t launch_pack(const uint8_t* route, int64_t rows, int32_t t_mask, uint64_t* words,
                       int32_t words_per_row, hipStream_t stream) {
  const int64_t n = rows * words_per_row;
  if (n == 0) return hipSuccess;
  pack_route_kernel<<<dim3(static_cast<unsigned>((n + 3) / 4)), dim3(256), 0, stream>>>(
      route, rows, t_mask, words, words_per_row);
  return hipGetLastError();
}

}  // namespace tilemix
