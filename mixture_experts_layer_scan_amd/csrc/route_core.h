// The router's per-token selection (see route.hip for the method), shared by
// the router kernels and the fused decode kernel that routes, sorts and runs
// GEMM1 in one launch.
#pragma once

#include "moe_common.h"

namespace moe {
namespace {

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// The better of (v, i) and the pair DPP control `ctrl` brings from another
// lane of the same 16-lane row (every lane of the row takes part).
template <int CTRL>
__device__ __forceinline__ void dpp_best(float& v, int& i) {
  const float ov = __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(0, i, CTRL, 0xF, 0xF, false);
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

// Wave-wide best pair under `better`, returned in every lane.
__device__ __forceinline__ void wave_best(float& v, int& i) {
  dpp_best<0xB1>(v, i);   // quad_perm [1, 0, 3, 2]
  dpp_best<0x4E>(v, i);   // quad_perm [2, 3, 0, 1]
  dpp_best<0x141>(v, i);  // row_half_mirror
  dpp_best<0x140>(v, i);  // row_mirror
  float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 1; r < kWave / 16; ++r) {
    const float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r));
    const int ri = __builtin_amdgcn_readlane(i, 16 * r);
    if (better(rv, ri, bv, bi)) {
      bv = rv;
      bi = ri;
    }
  }
  v = bv;
  i = bi;
}

// Routes token t with the whole wave; returns the selected expert id in lanes
// 0..k-1 (-1 in the other lanes) and, with `store`, writes the ids and
// weights of row t.
template <int EPL>
__device__ __forceinline__ int route_token(const float* __restrict__ logits, int64_t t, int E,
                                           int k, int score_fn, int renormalize, float rsf,
                                           int32_t* __restrict__ ids, float* __restrict__ w,
                                           uint16_t* __restrict__ w_bf16, bool store = true) {
  const int lane = lane_id();
  const float* row = logits + t * E;

  float v[EPL];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * kWave + lane;
    v[i] = (e < E) ? row[e] : -INFINITY;
    if (e >= E) taken |= 1u << i;
  }

  float my_v = -INFINITY;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = i * kWave + lane;
      if (!((taken >> i) & 1u) && better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
    wave_best(bv, bi);
    if (bi < E && (bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    if (lane == j) {
      my_v = bv;
      my_id = bi;
    }
  }

  // Scores of the selected experts (lanes < k) and the normaliser.
  const bool sel = lane < k;
  const float vmax = __shfl(my_v, 0, kWave);  // the first pick is the largest logit
  float p = 0.0f;
  if (score_fn == 0) {
    p = sel ? expf(my_v - vmax) : 0.0f;
  } else {
    p = sel ? 1.0f / (1.0f + expf(-my_v)) : 0.0f;
  }
  float denom = 1.0f;
  if (renormalize) {
    float s = p;
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, kWave);
    denom = s;
  } else if (score_fn == 0) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = i * kWave + lane;
      if (e < E) s += expf(v[i] - vmax);
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, kWave);
    denom = s;
  }
  if (sel && store) {
    const float wt = p / denom * rsf;
    ids[t * k + lane] = my_id;
    w[t * k + lane] = wt;
    if (w_bf16) w_bf16[t * k + lane] = f32_to_bf16(wt);
  }
  return sel ? my_id : -1;
}

// The local experts (or -1) of the experts whose logits lane l holds (l,
// l + 64, ...), loaded once per wave beside the logits, so that a pick's
// local expert needs no further memory round trip.
template <int EPL>
__device__ __forceinline__ void load_local_map(const int32_t* __restrict__ emap, int E, int E_l,
                                               int (&em)[EPL]) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * kWave + lane;
    const int l = e < E ? (emap ? emap[e] : e) : -1;
    em[i] = (l >= 0 && l < E_l) ? l : -1;
  }
}

// Local expert of pick id (from route_token; -1 for none): its entry sits in
// lane id % 64, register id / 64.  Every lane of the wave takes part.
template <int EPL>
__device__ __forceinline__ int local_of_pick(const int (&em)[EPL], int id, int E) {
  int l = -1;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int v = __shfl(em[i], id & (kWave - 1), kWave);
    if ((id >> 6) == i) l = v;
  }
  return (id >= 0 && id < E) ? l : -1;
}

}  // namespace
}  // namespace moe
