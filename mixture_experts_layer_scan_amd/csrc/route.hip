// Router: top-k experts per token and their weights (the [Router] stage of
// vLLM's modular fused-MoE kernel; the weights carry the routed scaling factor
// as the expert_weights comment of vLLM's MoE output contract describes).
//
// One wave per token.  Lane l holds logits l, l+64, l+128, ... in registers.
// Each of the k rounds takes a wave-wide argmax under the order
// (logit descending, expert id ascending): four DPP steps give every lane of
// each 16-lane row its row's best (swap within pairs, within quads, mirror
// within 8, mirror within 16), and the four rows' bests are read into scalar
// registers and compared there, so every lane ends the round with the same
// winner; the winning element is marked taken.  (DPP moves are register
// operations; a shuffle through the LDS crossbar costs a round trip per step.)
// Lane j keeps the j-th winner, so the k results end up in lanes 0..k-1 and
// are stored with one coalesced write.  Selection compares fp32 logits only
// (no arithmetic), so the chosen ids are exact.
#include "permute_core.h"
#include "route_core.h"

namespace moe {
namespace {

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int64_t T, int E, int k, int score_fn,
                                                         int renormalize, float rsf,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ w,
                                                         uint16_t* __restrict__ w_bf16) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // whole wave leaves together
  route_token<EPL>(logits, t, E, k, score_fn, renormalize, rsf, ids, w, w_bf16);
}

// Router and Permute of a small batch in one workgroup: wave w routes tokens
// w, w + 16, ... and keeps their local experts in LDS, then the workgroup
// runs the same counting sort as the permute kernel on them.  The map,
// offsets and inverse map equal those of the two separate kernels.
template <int EPL>
__global__ __launch_bounds__(kPermuteThreads) void route_permute_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int score_fn, int renormalize,
    float rsf, int32_t* __restrict__ ids, float* __restrict__ w, uint16_t* __restrict__ w_bf16,
    const int32_t* __restrict__ emap, int E_l, int32_t* __restrict__ map,
    int32_t* __restrict__ offsets, int32_t* __restrict__ inv, int64_t R_pad, int batch_m) {
  extern __shared__ int32_t smem[];
  int32_t* s_local = smem + sort_lds_bytes(E_l) / sizeof(int32_t);  // [T * k]
  const int lane = lane_id();
  if (threadIdx.x / kWave < T) {
    int em[EPL];
    load_local_map<EPL>(emap, E, E_l, em);
    for (int64_t t = threadIdx.x / kWave; t < T; t += kPermuteWaves) {
      const int id = route_token<EPL>(logits, t, E, k, score_fn, renormalize, rsf, ids, w, w_bf16);
      const int l = local_of_pick<EPL>(em, id, E);
      if (lane < k) s_local[t * k + lane] = l;
    }
  }
  __syncthreads();
  counting_sort(LdsRoutes{s_local}, T * k, E_l, map, offsets, inv, R_pad, batch_m, smem, 0, 1);
}

template <int EPL>
hipError_t launch_epl(const float* logits, int64_t T, int E, int k, int score_fn, int renorm,
                      float rsf, int32_t* ids, float* w, uint16_t* w_bf16, hipStream_t s) {
  const int per_block = 4;
  const int64_t blocks = (T + per_block - 1) / per_block;
  hipLaunchKernelGGL(route_topk_kernel<EPL>, dim3(static_cast<unsigned>(blocks)),
                     dim3(per_block * kWave), 0, s, logits, T, E, k, score_fn, renorm, rsf, ids,
                     w, w_bf16);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k, int score_fn,
                             int renormalize, float rsf, int32_t* ids, float* w,
                             uint16_t* w_bf16, hipStream_t s) {
  const int epl = (E + kWave - 1) / kWave;
  if (epl <= 1) return launch_epl<1>(logits, T, E, k, score_fn, renormalize, rsf, ids, w, w_bf16, s);
  if (epl <= 2) return launch_epl<2>(logits, T, E, k, score_fn, renormalize, rsf, ids, w, w_bf16, s);
  if (epl <= 4) return launch_epl<4>(logits, T, E, k, score_fn, renormalize, rsf, ids, w, w_bf16, s);
  if (epl <= 8) return launch_epl<8>(logits, T, E, k, score_fn, renormalize, rsf, ids, w, w_bf16, s);
  return launch_epl<16>(logits, T, E, k, score_fn, renormalize, rsf, ids, w, w_bf16, s);
}

namespace {
template <int EPL>
hipError_t launch_merged(const float* logits, int64_t T, int E, int k, int score_fn, int renorm,
                         float rsf, int32_t* ids, float* w, uint16_t* w_bf16, const int32_t* emap,
                         int E_l, int32_t* map, int32_t* offsets, int32_t* inv, int64_t R_pad,
                         int batch_m, hipStream_t s) {
  const size_t lds = sort_lds_bytes(E_l) + sizeof(int32_t) * T * k;
  static bool attr_set[kMaxDevices] = {};
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(route_permute_kernel<EPL>),
                                    80 * 1024, attr_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_permute_kernel<EPL>, dim3(1), dim3(kPermuteThreads), lds, s, logits, T,
                     E, k, score_fn, renorm, rsf, ids, w, w_bf16, emap, E_l, map, offsets, inv,
                     R_pad, batch_m);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_route_permute(const float* logits, int64_t T, int E, int k, int score_fn,
                                int renormalize, float rsf, int32_t* ids, float* w,
                                uint16_t* w_bf16, const int32_t* emap, int E_l, int32_t* map,
                                int32_t* offsets, int32_t* inv, int64_t R_pad, int batch_m,
                                hipStream_t s) {
  if (T > kRoutePermuteMaxT || T == 0) {
    hipError_t e = hipSuccess;
    if (T > 0) e = launch_route_topk(logits, T, E, k, score_fn, renormalize, rsf, ids, w, w_bf16, s);
    if (e != hipSuccess) return e;
    return launch_permute(ids, emap, T, k, E, E_l, map, offsets, inv, R_pad, s, batch_m);
  }
  const int epl = (E + kWave - 1) / kWave;
#define MOE_MERGED(N)                                                                          \
  return launch_merged<N>(logits, T, E, k, score_fn, renormalize, rsf, ids, w, w_bf16, emap, E_l, \
                          map, offsets, inv, R_pad, batch_m, s)
  if (epl <= 1) MOE_MERGED(1);
  if (epl <= 2) MOE_MERGED(2);
  if (epl <= 4) MOE_MERGED(4);
  if (epl <= 8) MOE_MERGED(8);
  MOE_MERGED(16);
#undef MOE_MERGED
}

}  // namespace moe
