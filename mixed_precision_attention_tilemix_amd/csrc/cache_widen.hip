// Pre-pass of the fused prefill over an INT8 K/V cache (TileMix paper, Section 4.3: the FP16
// path of a tile group over an INT8 cache works on the dequantized keys and values): K8 widened
// to an exact fp16 copy (the FP16-routed score tiles multiply in k_scale after the dot product)
// and V dequantized to fp16(v_scale * v8), both in the cache's [token, KV head, head_dim] layout,
// which the fused kernel streams like fp16 K and V. HBM-bound: one read of the cache, two writes.
#include "device_types.h"
#include "launch.h"

namespace tilemix {
namespace {

template <int D>
__global__ __launch_bounds__(256) void cache_widen_kernel(const FwdArgs a) {
  constexpr int CPR = D / 8;  // 8-element chunks per (token, head) row
  const int64_t n = a.total_k * a.hkv * CPR;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t row = i / CPR;  // token * hkv + head
    const int64_t tk = row / a.hkv;
    const int hk = static_cast<int>(row % a.hkv);
    const int2v v8 = reinterpret_cast<const int2v*>(a.v8)[i];
    const int2v k8 = reinterpret_cast<const int2v*>(a.k8)[i];
    const float vs = a.v_scale[static_cast<int64_t>(hk) * a.total_k + tk];
    const int8_t* vb = reinterpret_cast<const int8_t*>(&v8);
    const int8_t* kb = reinterpret_cast<const int8_t*>(&k8);
    half8v vh, kh;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      vh[e] = static_cast<_Float16>(static_cast<float>(vb[e]) * vs);
      kh[e] = static_cast<_Float16>(kb[e]);
    }
    reinterpret_cast<half8v*>(a.v16_ws)[i] = vh;
    reinterpret_cast<half8v*>(a.k16_ws)[i] = kh;
  }
}

}  // namespace

hipError_t launch_cache_widen(const FwdArgs& a, int32_t head_dim, hipStream_t stream) {
  const int64_t chunks = a.total_k * a.hkv * (head_dim / 8);
  if (chunks == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>(chunks / 256 + 1 < 8192 ? chunks / 256 + 1 : 8192);
  if (head_dim == 128)
    cache_widen_kernel<128><<<blocks, dim3(256), 0, stream>>>(a);
  else
    cache_widen_kernel<64><<<blocks, dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace tilemix
