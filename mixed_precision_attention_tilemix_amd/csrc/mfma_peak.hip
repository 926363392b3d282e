// Measured matrix-core peak of the GPU this runs on, for the roofline of the benchmark: a grid of
// wavefronts that each issue long runs of independent 32x32 MFMAs (the two shapes the fused
// prefill kernel uses: v_mfma_i32_32x32x32_i8 and v_mfma_f32_32x32x16_f16) with nothing else in
// the loop. Dense rate = MFMAs issued x flops per MFMA / launch time. Built as a separate
// library (libtilemix_peak.so) that only the benchmark loads; not part of the attention path.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int16v __attribute__((ext_vector_type(16)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));

constexpr int kChains = 4;  // independent accumulators per wavefront: keeps the pipe full

template <bool I8>
__global__ __launch_bounds__(256) void mfma_peak_kernel(float* out, int iters) {
  const int tid = threadIdx.x;
  float sum = 0.0f;
  if constexpr (I8) {
    const int4v a = {tid, tid + 1, tid + 2, tid + 3};
    const int4v b = {1, 2, 3, tid};
    int16v c[kChains] = {};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < kChains; ++k) c[k] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[k], 0, 0, 0);
#pragma unroll
    for (int k = 0; k < kChains; ++k) sum += static_cast<float>(c[k][0]);
  } else {
    half8v a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = static_cast<_Float16>(1e-3f * (tid + e));
      b[e] = static_cast<_Float16>(1e-3f * e);
    }
    float16v c[kChains] = {};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < kChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[k], 0, 0, 0);
#pragma unroll
    for (int k = 0; k < kChains; ++k) sum += c[k][0];
  }
  out[static_cast<int64_t>(blockIdx.x) * blockDim.x + tid] = sum;
}

}  // namespace

// Launches `blocks` workgroups of 256 threads on `stream`; each wavefront issues
// iters * 4 MFMAs of the given kind (0: INT8 32x32x32, 1: FP16 32x32x16). out holds
// blocks * 256 floats. Returns 0, or the hipError_t of the launch.
extern "C" int tilemix_peak_mfma(int kind, int blocks, int iters, float* out, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0)
    mfma_peak_kernel<true><<<blocks, 256, 0, s>>>(out, iters);
  else
    mfma_peak_kernel<false><<<blocks, 256, 0, s>>>(out, iters);
  return static_cast<int>(hipGetLastError());
}

// MFMAs per wavefront per iteration, for the caller's flop count.
extern "C" int tilemix_peak_chains(void) { return kChains; }
