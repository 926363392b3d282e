// Key-tile layout shared by the V^T pre-pass and the fused kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tilemix {

constexpr int kKeyTile = 64;  // keys per tile of the fused kernel's inner loop

// A V^T tile is [head_dim rows][64 keys] fp16: row d occupies 128 bytes, split in eight 16-byte
// chunks of 8 consecutive keys; chunk c of row d is stored at position c ^ vt_swizzle(d), which
// spreads the 32 rows that one MFMA operand read touches over distinct LDS banks.
__device__ __forceinline__ int vt_swizzle(int d) { return (d >> 1) & 7; }

// Number of 64-key tiles of sequences [0, b): tiles never straddle sequences.
__device__ __forceinline__ int key_tiles_before(const int32_t* cu_k, int b) {
  int t = 0;
  for (int i = 0; i < b; ++i) t += (cu_k[i + 1] - cu_k[i] + kKeyTile - 1) / kKeyTile;
  return t;
}

// Upper bound of the number of 64-key tiles over all sequences (host side).
inline int64_t key_tiles_bound(int64_t total_k, int32_t batch) {
  return (total_k + kKeyTile - 1) / kKeyTile + batch;
}

}  // namespace tilemix
