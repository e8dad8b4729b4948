// Permute: the single-GPU part of [Quantize-Dispatch] of vLLM's modular
// fused-MoE kernel (prepare() with its expert_map and per-local-expert counts)
// producing the expanded_idx_to_permuted_idx map of vLLM's MoE output contract
// (int32, -1 for an expert that is not local).
//
// Deterministic stable counting sort (permute_core.h), one workgroup of 16
// waves per 1024 routes (at most 256 workgroups), each placing the routes of
// its own contiguous range of the expanded index x = t*k + j:
//   - every workgroup first counts all routes per local expert with integer
//     LDS atomics (their sums do not depend on the order), in total and
//     before its range, so the workgroups never wait for one another;
//   - wave w owns a contiguous run of the range and walks it 64 routes at a
//     time, loading the expert ids (and their expert-map entries) of 16 such
//     steps ahead with independent loads;
//   - per-wave counts, a column scan over the 16 waves and a block scan over
//     experts give every (wave, expert) pair its first output row;
//   - inside a step, lanes with equal local expert find each other with a
//     ballot per key bit (wave_match) and each takes the popcount of its
//     lower-lane peers as its rank, so the order within an expert is
//     ascending x.
// Batched experts format (batch_m > 0): expert L owns rows [L * batch_m,
// (L + 1) * batch_m); the same ranks place a route at L * batch_m + rank, or
// -1 past the capacity, and `offsets` receives the per-expert counts.
// Rows are then gathered token-major: each token row is read once and written
// to each of its (up to k) local slots with 16-byte accesses.  With
// apply_router_weight_on_input (prepare() applies the routing weights to the
// activations before dispatch) each slot receives bf16(w[t, j] * x[t]).
#include "permute_core.h"

namespace moe {
namespace {

__global__ __launch_bounds__(kPermuteThreads) void permute_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ emap, int64_t R, int E, int E_l,
    int32_t* __restrict__ map, int32_t* __restrict__ offsets, int32_t* __restrict__ inv,
    int64_t R_pad, int batch_m) {
  extern __shared__ int32_t smem[];
  counting_sort(GlobalRoutes{ids, emap, E, E_l}, R, E_l, map, offsets, inv, R_pad, batch_m, smem,
                static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
}

// x_perm[map[t, j], :] = x[t, :] for every local route of token t.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ x,
                                                          const int32_t* __restrict__ map,
                                                          int64_t T, int k, int H8,
                                                          uint4* __restrict__ x_perm) {
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const int32_t* m = map + t * k;
    const uint4* src = x + t * H8;
    for (int c = threadIdx.x; c < H8; c += blockDim.x) {
      const uint4 v = src[c];
      for (int j = 0; j < k; ++j) {
        const int32_t r = m[j];
        if (r >= 0) x_perm[static_cast<int64_t>(r) * H8 + c] = v;
      }
    }
  }
}

__global__ __launch_bounds__(256) void gather_scaled_rows_kernel(const uint4* __restrict__ x,
                                                                 const int32_t* __restrict__ map,
                                                                 const float* __restrict__ scale,
                                                                 int64_t T, int k, int H8,
                                                                 uint4* __restrict__ x_perm) {
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const int32_t* m = map + t * k;
    const uint4* src = x + t * H8;
    for (int c = threadIdx.x; c < H8; c += blockDim.x) {
      const uint4 v = src[c];
      const uint32_t p[4] = {v.x, v.y, v.z, v.w};
      for (int j = 0; j < k; ++j) {
        const int32_t r = m[j];
        if (r < 0) continue;
        const float w = scale[t * k + j];
        uint32_t q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          q[i] = pack_bf16x2(w * bf16_to_f32(static_cast<uint16_t>(p[i] & 0xFFFFu)),
                             w * bf16_to_f32(static_cast<uint16_t>(p[i] >> 16)));
        x_perm[static_cast<int64_t>(r) * H8 + c] = uint4{q[0], q[1], q[2], q[3]};
      }
    }
  }
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v0, int32_t step) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v0 + static_cast<int32_t>(i) * step;
}

__global__ void fill_u16_kernel(uint16_t* p, int64_t n, uint16_t v) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

}  // namespace

hipError_t launch_permute(const int32_t* ids, const int32_t* emap, int64_t T, int k, int E,
                          int E_l, int32_t* map, int32_t* offsets, int32_t* inv, int64_t R_pad,
                          hipStream_t s, int batch_m) {
  const size_t lds = sort_lds_bytes(E_l);
  static bool attr_set[kMaxDevices] = {};
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(permute_kernel), 80 * 1024,
                                    attr_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(permute_kernel, dim3(sort_blocks(T * k)), dim3(kPermuteThreads), lds, s, ids,
                     emap, T * k, E, E_l, map, offsets, inv, R_pad, batch_m);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* map, int64_t T, int k, int H,
                              const float* scale, void* x_perm, hipStream_t s) {
  const int64_t blocks = T < 8192 ? T : 8192;
  if (scale)
    hipLaunchKernelGGL(gather_scaled_rows_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256),
                       0, s, static_cast<const uint4*>(x), map, scale, T, k, H / 8,
                       static_cast<uint4*>(x_perm));
  else
    hipLaunchKernelGGL(gather_rows_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const uint4*>(x), map, T, k, H / 8,
                       static_cast<uint4*>(x_perm));
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v0, int32_t step, hipStream_t s) {
  const int64_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(static_cast<unsigned>(blocks > 0 ? blocks : 1)),
                     dim3(256), 0, s, p, n, v0, step);
  return hipGetLastError();
}

hipError_t launch_fill_u16(uint16_t* p, int64_t n, uint16_t v, hipStream_t s) {
  const int64_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  hipLaunchKernelGGL(fill_u16_kernel, dim3(static_cast<unsigned>(blocks > 0 ? blocks : 1)),
                     dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace moe
