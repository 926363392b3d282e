// Pre-pass of the fused prefill on its V^T path: every 64-key tile of V is written transposed
// ([head_dim][64]), in the chunk-swizzled order the fused kernel keeps in LDS, so that the kernel
// streams each V^T tile as one contiguous block and feeds the P.V product with single 16-byte LDS
// reads. With an INT8 K/V cache the same pass dequantizes V (fp16(v_scale * v8)) and widens K8 to
// an exact fp16 copy for the FP16-routed tiles. HBM-bound: one read and one write of V (and K).
#include "device_types.h"
#include "launch.h"
#include "tile_layout.h"

namespace tilemix {
namespace {

template <int D, bool KV8>
__global__ __launch_bounds__(256) void vt_pack_kernel(const FwdArgs a) {
  constexpr int T = kKeyTile;
  constexpr int CPR = D / 8;  // 8-element chunks per key row
  __shared__ _Float16 tile[T][D + 8];
  const int n = blockIdx.x, b = blockIdx.y, hk = blockIdx.z;
  // the fused kernel's work-queue counters start at zero (the fused kernel follows on the stream)
  if (a.sched != nullptr && n == 0 && b == 0 && hk == 0 && threadIdx.x < 8) a.sched[threadIdx.x] = 0;
  const int k_begin = a.cu_k[b];
  const int Lk = a.cu_k[b + 1] - k_begin;
  const int j0 = n * T;
  if (j0 >= Lk) return;
  const int tid = threadIdx.x;

  for (int ch = tid; ch < T * CPR; ch += 256) {
    const int row = ch / CPR, col = ch % CPR;
    const int key = j0 + row;
    half8v val = {};
    if (key < Lk) {
      const int64_t tk = k_begin + key;
      if (!KV8) {
        val = *reinterpret_cast<const half8v*>(a.v + tk * a.v_stride_tok + hk * a.v_stride_head + col * 8);
      } else {
        const int64_t base = (tk * a.hkv + hk) * D + col * 8;
        const int2v v8 = *reinterpret_cast<const int2v*>(a.v8 + base);
        const int2v k8 = *reinterpret_cast<const int2v*>(a.k8 + base);
        const float vs = a.v_scale[static_cast<int64_t>(hk) * a.total_k + tk];
        const int8_t* vb = reinterpret_cast<const int8_t*>(&v8);
        const int8_t* kb = reinterpret_cast<const int8_t*>(&k8);
        half8v kh;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          val[e] = static_cast<_Float16>(static_cast<float>(vb[e]) * vs);
          kh[e] = static_cast<_Float16>(kb[e]);
        }
        *reinterpret_cast<half8v*>(a.k16_ws + base) = kh;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[row][col * 8 + e] = val[e];
  }
  __syncthreads();

  const int64_t slot = static_cast<int64_t>(hk) * a.vt_tiles + key_tiles_before(a.cu_k, b) + n;
  _Float16* out = a.vt_ws + slot * (D * T);
  for (int ch = tid; ch < D * (T / 8); ch += 256) {
    const int d = ch / (T / 8), pos = ch % (T / 8);
    const int c = pos ^ vt_swizzle(d);
    half8v val;
#pragma unroll
    for (int e = 0; e < 8; ++e) val[e] = tile[8 * c + e][d];
    *reinterpret_cast<half8v*>(out + d * T + pos * 8) = val;
  }
}

template <int D, bool KV8>
hipError_t launch_t(const FwdArgs& a, int32_t batch, int32_t max_seqlen_k, hipStream_t stream) {
  const int n_tiles = (max_seqlen_k + kKeyTile - 1) / kKeyTile;
  if (n_tiles == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>(n_tiles), static_cast<unsigned>(batch), static_cast<unsigned>(a.hkv));
  vt_pack_kernel<D, KV8><<<grid, dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_vt_pack(const FwdArgs& a, int32_t batch, int32_t max_seqlen_k, int32_t head_dim,
                          bool kv_int8, hipStream_t stream) {
  if (head_dim == 128)
    return kv_int8 ? launch_t<128, true>(a, batch, max_seqlen_k, stream)
                   : launch_t<128, false>(a, batch, max_seqlen_k, stream);
  return kv_int8 ? launch_t<64, true>(a, batch, max_seqlen_k, stream)
                 : launch_t<64, false>(a, batch, max_seqlen_k, stream);
}

}  // namespace tilemix
