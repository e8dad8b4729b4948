// Finalize = Unpermute + Combine (finalize() of vLLM's modular fused-MoE
// kernel: apply the routing weights to the unweighted expert rows and reduce
// over top-k; MoEOutput of vLLM's MoE output contract: the routed scaling
// factor multiplies the routed sum before the shared-expert add).
//
//   out[t, :] = rsf_fin * sum_{j ascending, map[t,j] >= 0} w[t,j] * y[map[t,j], :]
//               + shared[t, :]
//
// One workgroup per token (grid-stride); each thread owns 8 consecutive
// columns, so every access is a 16-byte load or store.  The routes of the
// token (map and weights, k <= 32) are staged once in LDS.
// Entries of -1 are skipped, so rows the map never names are never read.
// Accumulation is fp32 in j order, rounded once to bf16.
#include "moe_common.h"

namespace moe {
namespace {

template <bool W_BF16>
__global__ __launch_bounds__(256) void finalize_kernel(const uint4* __restrict__ y,
                                                       const void* __restrict__ wts,
                                                       const int32_t* __restrict__ map,
                                                       int64_t T, int k, int H8, float rsf_fin,
                                                       const uint4* shared, uint4* out) {
  __shared__ int32_t s_row[32];
  __shared__ float s_w[32];
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    __syncthreads();  // the previous token's routes are no longer read
    if (threadIdx.x < k) {
      s_row[threadIdx.x] = map[t * k + threadIdx.x];
      s_w[threadIdx.x] = W_BF16
          ? bf16_to_f32(static_cast<const uint16_t*>(wts)[t * k + threadIdx.x])
          : static_cast<const float*>(wts)[t * k + threadIdx.x];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < H8; c += blockDim.x) {
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
      for (int j = 0; j < k; ++j) {
        const int32_t r = s_row[j];
        if (r < 0) continue;
        const float wj = s_w[j];
        const uint4 v = y[static_cast<int64_t>(r) * H8 + c];
        const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += wj * bf16_to_f32(static_cast<uint16_t>(p[i] & 0xFFFFu));
          acc[2 * i + 1] += wj * bf16_to_f32(static_cast<uint16_t>(p[i] >> 16));
        }
      }
      float add[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) add[i] = 0.0f;
      if (shared) {
        const uint4 sv = shared[t * H8 + c];
        const uint32_t p[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          add[2 * i] = bf16_to_f32(static_cast<uint16_t>(p[i] & 0xFFFFu));
          add[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(p[i] >> 16));
        }
      }
      uint4 o;
      o.x = pack_bf16x2(rsf_fin * acc[0] + add[0], rsf_fin * acc[1] + add[1]);
      o.y = pack_bf16x2(rsf_fin * acc[2] + add[2], rsf_fin * acc[3] + add[3]);
      o.z = pack_bf16x2(rsf_fin * acc[4] + add[4], rsf_fin * acc[5] + add[5]);
      o.w = pack_bf16x2(rsf_fin * acc[6] + add[6], rsf_fin * acc[7] + add[7]);
      out[t * H8 + c] = o;
    }
  }
}

}  // namespace

hipError_t launch_finalize(const void* y, const void* w, int w_is_bf16, const int32_t* map,
                           int64_t T, int k, int H, float rsf_fin, const void* shared, void* out,
                           hipStream_t s) {
  const int H8 = H / 8;
  const int threads = H8 >= 256 ? 256 : ((H8 + 63) / 64) * 64;
  const int64_t blocks = T < 16384 ? T : 16384;
  if (w_is_bf16)
    hipLaunchKernelGGL(finalize_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(threads),
                       0, s, static_cast<const uint4*>(y), w, map, T, k, H8, rsf_fin,
                       static_cast<const uint4*>(shared), static_cast<uint4*>(out));
  else
    hipLaunchKernelGGL(finalize_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(threads),
                       0, s, static_cast<const uint4*>(y), w, map, T, k, H8, rsf_fin,
                       static_cast<const uint4*>(shared), static_cast<uint4*>(out));
  return hipGetLastError();
}

}  // namespace moe
