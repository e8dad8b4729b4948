// Finalize = Unpermute + Combine (finalize() of vLLM's modular fused-MoE
// kernel: apply the routing weights to the unweighted expert rows and reduce
// over top-k; MoEOutput of vLLM's MoE output contract: the routed scaling
// factor multiplies the routed sum before the shared-expert add).
//
//   out[t, :] = rsf_fin * sum_{j ascending, map[t,j] >= 0} w[t,j] * y[map[t,j], :]
//               + shared[t, :]
//
// One workgroup per token (grid-stride); each thread owns 8 consecutive
// columns, so every access is a 16-byte load or store.  With few tokens the
// columns of a token are split over gridDim.y workgroups, so a decode batch
// still spreads over the chip.  The routes of the token (map and weights,
// k <= 32) are staged once in LDS; a thread issues the loads of up to 8
// routes before it adds any of them, so their latencies overlap.
// Entries of -1, and entries at or past the caller's row count of y, are
// skipped, so no row outside y is ever read.
// Accumulation is fp32 in j order, rounded once to bf16.  Without weights
// (NULL) every route counts once: finalize() with apply_router_weight_on_input,
// whose weights were applied to the inputs.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kRouteBatch = 8;  // route rows loaded before they are added

// acc[0..8) = sum over j ascending with row s_row[j] >= 0 of s_w[j] * y[row, 8c .. 8c+7]
// (rows of -1 add nothing; the loads of a batch of routes are in flight together)
__device__ __forceinline__ void sum_routes(const uint4* __restrict__ y, int H8, int c, int k,
                                           const int32_t* s_row, const float* s_w, float* acc) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  for (int j0 = 0; j0 < k; j0 += kRouteBatch) {
    uint4 v[kRouteBatch];
#pragma unroll
    for (int jj = 0; jj < kRouteBatch; ++jj) {
      const int32_t r = j0 + jj < k ? s_row[j0 + jj] : -1;
      v[jj] = r >= 0 ? y[static_cast<int64_t>(r) * H8 + c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int jj = 0; jj < kRouteBatch; ++jj) {
      if (j0 + jj >= k || s_row[j0 + jj] < 0) continue;
      const float wj = s_w[j0 + jj];
      const uint32_t p[4] = {v[jj].x, v[jj].y, v[jj].z, v[jj].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += wj * bf16_to_f32(static_cast<uint16_t>(p[i] & 0xFFFFu));
        acc[2 * i + 1] += wj * bf16_to_f32(static_cast<uint16_t>(p[i] >> 16));
      }
    }
  }
}

template <bool W_BF16>
__global__ __launch_bounds__(256) void finalize_kernel(const uint4* __restrict__ y,
                                                       const void* __restrict__ wts,
                                                       const int32_t* __restrict__ map,
                                                       int64_t y_rows, int64_t T, int k, int H8,
                                                       float rsf_fin, const uint4* shared,
                                                       uint4* out) {
  __shared__ int32_t s_row[32];
  __shared__ float s_w[32];
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    __syncthreads();  // the previous token's routes are no longer read
    if (threadIdx.x < k) {
      const int32_t r = map[t * k + threadIdx.x];
      s_row[threadIdx.x] = r < y_rows ? r : -1;
      s_w[threadIdx.x] = !wts ? 1.0f
          : W_BF16 ? bf16_to_f32(static_cast<const uint16_t*>(wts)[t * k + threadIdx.x])
                   : static_cast<const float*>(wts)[t * k + threadIdx.x];
    }
    __syncthreads();
    for (int c = blockIdx.y * blockDim.x + threadIdx.x; c < H8; c += gridDim.y * blockDim.x) {
      float acc[8];
      sum_routes(y, H8, c, k, s_row, s_w, acc);
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

// Fused tail (MoEOutput of vLLM's MoE output contract: the next layer's
// RMSNorm is the consumer that folds the open reduction into itself):
//
//   z[t, :] = rsf_fin * sum_j w[t,j] * y[map[t,j], :] + shared[t, :] + residual[t, :]
//   residual[t, :] = bf16(z[t, :])                            (in place)
//   out[t, :] = bf16(z[t, :] / sqrt(mean(z[t, :]^2) + eps) * gamma)
//
// The norm uses the fp32 z, before the residual's rounding.  One workgroup
// per token: pass 1 forms z (as finalize does), writes the residual, keeps z
// in LDS and sums its squares; a block reduction gives 1/rms; pass 2 writes
// out.  H <= kTailMaxH (z of one token in LDS).
template <bool W_BF16>
__global__ __launch_bounds__(256) void finalize_norm_kernel(
    const uint4* __restrict__ y, const void* __restrict__ wts, const int32_t* __restrict__ map,
    int64_t y_rows, int64_t T, int k, int H8, float rsf_fin, const uint4* shared, uint4* residual,
    const uint4* __restrict__ gamma, float eps, uint4* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) float s_z[];  // [8 * H8]
  __shared__ int32_t s_row[32];
  __shared__ float s_w[32];
  __shared__ float s_part[16];
  const int nw = (blockDim.x + kWave - 1) / kWave;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    __syncthreads();  // the previous token's routes and sums are no longer read
    if (threadIdx.x < k) {
      const int32_t r = map[t * k + threadIdx.x];
      s_row[threadIdx.x] = r < y_rows ? r : -1;
      s_w[threadIdx.x] = !wts ? 1.0f
          : W_BF16 ? bf16_to_f32(static_cast<const uint16_t*>(wts)[t * k + threadIdx.x])
                   : static_cast<const float*>(wts)[t * k + threadIdx.x];
    }
    __syncthreads();
    float ss = 0.0f;
    for (int c = threadIdx.x; c < H8; c += blockDim.x) {
      float acc[8];
      sum_routes(y, H8, c, k, s_row, s_w, acc);
      float z[8];
      const uint4 rv = residual[t * H8 + c];
      const uint4 sv = shared ? shared[t * H8 + c] : make_uint4(0, 0, 0, 0);
      const uint32_t rp[4] = {rv.x, rv.y, rv.z, rv.w};
      const uint32_t sp[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[2 * i] = rsf_fin * acc[2 * i] + bf16_to_f32(static_cast<uint16_t>(sp[i] & 0xFFFFu)) +
                   bf16_to_f32(static_cast<uint16_t>(rp[i] & 0xFFFFu));
        z[2 * i + 1] = rsf_fin * acc[2 * i + 1] + bf16_to_f32(static_cast<uint16_t>(sp[i] >> 16)) +
                       bf16_to_f32(static_cast<uint16_t>(rp[i] >> 16));
      }
      uint4 o;
      o.x = pack_bf16x2(z[0], z[1]);
      o.y = pack_bf16x2(z[2], z[3]);
      o.z = pack_bf16x2(z[4], z[5]);
      o.w = pack_bf16x2(z[6], z[7]);
      residual[t * H8 + c] = o;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        s_z[c * 8 + i] = z[i];
        ss += z[i] * z[i];
      }
    }
    // block sum of squares: wave butterflies, then the wave totals in order
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, kWave);
    if (lane_id() == 0) s_part[threadIdx.x / kWave] = ss;
    __syncthreads();
    float total = 0.0f;
    for (int i = 0; i < nw; ++i) total += s_part[i];
    const float inv = 1.0f / sqrtf(total / static_cast<float>(8 * H8) + eps);
    for (int c = threadIdx.x; c < H8; c += blockDim.x) {
      const uint4 gv = gamma[c];
      const uint32_t gp[4] = {gv.x, gv.y, gv.z, gv.w};
      float v[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = s_z[c * 8 + 2 * i] * inv * bf16_to_f32(static_cast<uint16_t>(gp[i] & 0xFFFFu));
        v[2 * i + 1] = s_z[c * 8 + 2 * i + 1] * inv * bf16_to_f32(static_cast<uint16_t>(gp[i] >> 16));
      }
      uint4 o;
      o.x = pack_bf16x2(v[0], v[1]);
      o.y = pack_bf16x2(v[2], v[3]);
      o.z = pack_bf16x2(v[4], v[5]);
      o.w = pack_bf16x2(v[6], v[7]);
      out[t * H8 + c] = o;
    }
  }
}

}  // namespace

hipError_t launch_finalize_add_rmsnorm(const void* y, int64_t y_rows, const void* w, int w_is_bf16,
                                       const int32_t* map, int64_t T, int k, int H, float rsf_fin,
                                       const void* shared, void* residual, const void* gamma,
                                       float eps, void* out, hipStream_t s) {
  const int H8 = H / 8;
  const int threads = H8 >= 256 ? 256 : ((H8 + 63) / 64) * 64;
  const int64_t blocks = T < 16384 ? T : 16384;
  const size_t lds = sizeof(float) * static_cast<size_t>(H);
  static bool attr_set[2][kMaxDevices] = {};
  const void* fn = w_is_bf16 ? reinterpret_cast<const void*>(finalize_norm_kernel<true>)
                             : reinterpret_cast<const void*>(finalize_norm_kernel<false>);
  hipError_t e = ensure_dynamic_lds(fn, static_cast<int>(sizeof(float) * kTailMaxH),
                                    attr_set[w_is_bf16 ? 1 : 0]);
  if (e != hipSuccess) return e;
  if (w_is_bf16)
    hipLaunchKernelGGL(finalize_norm_kernel<true>, dim3(static_cast<unsigned>(blocks)),
                       dim3(threads), lds, s, static_cast<const uint4*>(y), w, map, y_rows, T, k, H8,
                       rsf_fin, static_cast<const uint4*>(shared), static_cast<uint4*>(residual),
                       static_cast<const uint4*>(gamma), eps, static_cast<uint4*>(out));
  else
    hipLaunchKernelGGL(finalize_norm_kernel<false>, dim3(static_cast<unsigned>(blocks)),
                       dim3(threads), lds, s, static_cast<const uint4*>(y), w, map, y_rows, T, k, H8,
                       rsf_fin, static_cast<const uint4*>(shared), static_cast<uint4*>(residual),
                       static_cast<const uint4*>(gamma), eps, static_cast<uint4*>(out));
  return hipGetLastError();
}

hipError_t launch_finalize(const void* y, int64_t y_rows, const void* w, int w_is_bf16,
                           const int32_t* map, int64_t T, int k, int H, float rsf_fin,
                           const void* shared, void* out, hipStream_t s) {
  const int H8 = H / 8;
  const int threads = H8 >= 256 ? 256 : ((H8 + 63) / 64) * 64;
  const int64_t blocks = T < 16384 ? T : 16384;
  // few tokens: each token's columns over several workgroups (one column
  // chunk per thread), so a decode batch fills more than a few CUs
  const int split = T < 1024 ? (H8 + threads - 1) / threads : 1;
  const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(split));
  if (w_is_bf16)
    hipLaunchKernelGGL(finalize_kernel<true>, grid, dim3(threads),
                       0, s, static_cast<const uint4*>(y), w, map, y_rows, T, k, H8, rsf_fin,
                       static_cast<const uint4*>(shared), static_cast<uint4*>(out));
  else
    hipLaunchKernelGGL(finalize_kernel<false>, grid, dim3(threads),
                       0, s, static_cast<const uint4*>(y), w, map, y_rows, T, k, H8, rsf_fin,
                       static_cast<const uint4*>(shared), static_cast<uint4*>(out));
  return hipGetLastError();
}

}  // namespace moe
