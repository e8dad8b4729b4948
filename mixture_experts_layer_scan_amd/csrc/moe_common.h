// Shared device helpers and host launch declarations of the MoE HIP library.
// gfx950 (CDNA4) only: wave64, MFMA, 160 KiB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// ---- bf16 <-> fp32 (bit patterns in uint16_t) ------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even; NaN stays NaN (quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x & (kWave - 1)); }

// ---- GEMM1 activations: act(gate) * up ---------------------------------------
// silu(g) = g / (1 + e^-g); gelu(g) = g/2 * (1 + erf(g / sqrt 2)) (erf form).
// A clamp c > 0 first limits the gate to <= c and the up value to [-c, c].
// Kinds: 0 silu, 1 silu with clamp, 2 gelu (cl = +inf without a clamp).
enum : int { kActSilu = 0, kActGelu = 1 };

template <int KIND>
__device__ __forceinline__ float gated_act_k(float g, float u, float cl) {
  if constexpr (KIND == 0) {
    return g / (1.0f + __expf(-g)) * u;
  } else {
    g = fminf(g, cl);
    u = fminf(fmaxf(u, -cl), cl);
    if constexpr (KIND == 1) return g / (1.0f + __expf(-g)) * u;
    return 0.5f * g * (1.0f + erff(g * 0.7071067811865476f)) * u;
  }
}

__host__ __device__ __forceinline__ int act_kind(int act, float clamp) {
  return act == kActGelu ? 2 : (clamp > 0.0f ? 1 : 0);
}

__host__ __device__ __forceinline__ float act_limit(float clamp) {
  return clamp > 0.0f ? clamp : __builtin_huge_valf();
}

// Mask of lanes of this wave whose `key` equals this lane's, among lanes with
// `active` set (0 for an inactive lane).  key must lie in [0, 2^nbits).
__device__ __forceinline__ uint64_t wave_match(uint32_t key, bool active, int nbits) {
  uint64_t peers = __ballot(active);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1u;
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return active ? peers : 0ull;
}

// Inclusive prefix sum over the lanes of a wave.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// Exclusive prefix sum of one int per thread over a whole block of
// blockDim.x <= 1024 threads.  `scratch` holds >= 16 ints of LDS.  Returns the
// exclusive prefix; *total receives the block sum.  Contains __syncthreads().
__device__ __forceinline__ int block_exclusive_sum(int v, int* scratch, int* total) {
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int nw = (blockDim.x + kWave - 1) / kWave;
  const int inc = wave_inclusive_sum(v);
  if (lane == kWave - 1) scratch[w] = inc;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const int s = scratch[i];
    if (i < w) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

}  // namespace moe

// ---- host launchers (one per .hip file); each returns a hipError_t ----------
namespace moe {

struct GemmArgs {
  const void* a;          // bf16 [R_pad, K], or fp8 e4m3 [R_pad, K] when a_scales is set
  const void* w;          // bf16 [E_l, N_total, K], packed e2m1 [E_l, N_total, K/2], or
                          // fp8 e4m3 [E_l, N_total, K]
  const void* w_scales;   // NULL (bf16), E8M0 u8 [E_l, N_total, K/32] (MXFP4), or fp32
                          // [E_l, N_total] per output channel (fp8)
  const int32_t* offsets; // [E_l + 1], or the E_l row counts when batch_m > 0
  int E_l;
  int K;
  int N_out;              // output columns (I when gated, else N)
  int gated;              // 1: GEMM1 with silu(gate) * up, N_total = 2 * N_out
  int64_t R_pad;
  void* c;                // bf16 [R_pad, N_out]
  // optional scratch for split reductions (256-byte aligned; NULL: no split)
  void* split_ws = nullptr;
  size_t split_ws_bytes = 0;
  int act = kActSilu;     // gated only: kActSilu or kActGelu
  float clamp = 0.0f;     // gated only: > 0 clamps gate and up first
  int batch_m = 0;        // > 0: batched experts format, expert e's rows start
                          // at e * batch_m and number min(offsets[e], batch_m)
  const float* a_scales = nullptr;  // fp8 activations: fp32 [R_pad], one per row
  bool w_mxfp4 = false;             // with fp8 activations: MXFP4 weights (else FP8)
  int a_terms = 1;                  // 2: two-term fp8 activations [R_pad, 2K] (MXFP4 weights)
  // gathered activations (bf16, FP8 or two-term FP8 with one scale per row):
  // a holds a_T token rows [a_T, K] and permuted row r reads token
  // a_inv[r] / a_k (a_inv: the permute's inverse map), with that token's scale
  const int32_t* a_inv = nullptr;
  int a_k = 1;
  int64_t a_T = 0;
  // > 0: blockwise FP8 (FP8 weights): a_scales holds one scale per row and
  // 128 k, k-block-major [K / 128][a_ld]; w_scales one per 128 x 128 weight
  // block, [E_l][N_total / 128][K / 128]
  int64_t a_ld = 0;
};

// Scratch bytes with which a grouped GEMM of R_pad rows may split its
// reduction into the most pieces it uses (0 when it never splits: more than
// 65535 rows, or a budget of 64 MiB exceeded by two slices).
size_t gemm_split_ws_bytes(int64_t R_pad, int N_total);

hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k, int score_fn,
                             int renormalize, float rsf, int32_t* ids, float* w,
                             uint16_t* w_bf16, hipStream_t s);
// batch_m > 0: batched experts format (rows [L * batch_m, ...) per expert,
// offsets receives the E_l per-expert counts; inv must be NULL)
hipError_t launch_permute(const int32_t* ids, const int32_t* emap, int64_t T, int k, int E,
                          int E_l, int32_t* map, int32_t* offsets, int32_t* inv, int64_t R_pad,
                          hipStream_t s, int batch_m = 0);
// Router and the permute map in one launch for T <= kRoutePermuteMaxT (one
// workgroup, one token per wave); larger batches launch the router and the
// permute kernels (the router then spreads its tokens over many compute
// units: in one workgroup every further token per wave costs about 6 us).
// Results equal launch_route_topk followed by launch_permute.
constexpr int64_t kRoutePermuteMaxT = 16;
hipError_t launch_route_permute(const float* logits, int64_t T, int E, int k, int score_fn,
                                int renormalize, float rsf, int32_t* ids, float* w,
                                uint16_t* w_bf16, const int32_t* emap, int E_l, int32_t* map,
                                int32_t* offsets, int32_t* inv, int64_t R_pad, int batch_m,
                                hipStream_t s);
// x_perm[map[t, j]] = x[t], or bf16(scale[t, j] * x[t]) when scale is given
hipError_t launch_gather_rows(const void* x, const int32_t* map, int64_t T, int k, int H,
                              const float* scale, void* x_perm, hipStream_t s);
hipError_t launch_grouped_gemm(const GemmArgs& g, int64_t max_rows, hipStream_t s);
// Grouped GEMM for experts with a few rows each (bf16 weights and rows): one
// workgroup per slice of 16 weight rows over the whole k-range, no split
// reduction.  decode_gemm_fits: K a multiple of 256, N_out of 8 (gated) or 16.
bool decode_gemm_fits(const GemmArgs& g);
hipError_t launch_decode_gemm(const GemmArgs& g, hipStream_t s);
// The same for FP8 E4M3 rows and weights with per-row and per-weight-row
// scales (no MXFP4, two-term or blockwise): K a multiple of 512.
bool decode_gemm_fp8_fits(const GemmArgs& g);
hipError_t launch_decode_gemm_fp8(const GemmArgs& g, hipStream_t s);
// launch_grouped_gemm(g, max_rows) runs the decode kernel
bool gemm_picks_decode(const GemmArgs& g, int64_t max_rows);
// Router, permute map (inverse map included) and gathered GEMM1 in one launch
// (g: the gathered bf16 GEMM1 of the decode kernel, its a_inv and offsets
// the buffers to fill).  Fits: T <= 8 tokens, T * k <= 64 routes, E <= 1024.
bool decode_route_gemm1_fits(const GemmArgs& g, int64_t T, int E, int k);
hipError_t launch_decode_route_gemm1(const float* logits, int64_t T, int E, int k, int score_fn,
                                     int renormalize, float rsf, int32_t* ids, float* wts,
                                     uint16_t* w_bf16, const int32_t* emap, int32_t* map,
                                     int32_t* offsets, int32_t* inv, int64_t R_pad,
                                     const GemmArgs& g, hipStream_t s);
// w == NULL: every weight is 1 (the weights were applied to the inputs);
// y has y_rows rows, map entries at or past them count as -1
hipError_t launch_finalize(const void* y, int64_t y_rows, const void* w, int w_is_bf16,
                           const int32_t* map, int64_t T, int k, int H, float rsf_fin,
                           const void* shared, void* out, hipStream_t s);
constexpr int kTailMaxH = 16384;  // the fused tail keeps one token's fp32 row in LDS
hipError_t launch_finalize_add_rmsnorm(const void* y, int64_t y_rows, const void* w, int w_is_bf16,
                                       const int32_t* map, int64_t T, int k, int H, float rsf_fin,
                                       const void* shared, void* residual, const void* gamma,
                                       float eps, void* out, hipStream_t s);
// FP8 E4M3 rows: q [rows, H] codes and one fp32 scale per row, from bf16 rows
// (times mult[r] rounded to bf16 when given); static_scale NULL: per-row
// dynamic scales; row_count (device) NULL: all rows, else rows < *row_count.
// terms 2: two-term codes, [rows, 2H] bytes (per 64 k: the first term's 64
// codes, then the second's), dynamic scales only
hipError_t launch_quantize_fp8(const void* x, int64_t rows, int H, const float* static_scale,
                               const float* mult, const int32_t* row_count, void* q,
                               float* scales, hipStream_t s, int terms = 1);
// groups > 0: blockwise scales, group-major [groups, T] in and [groups, R_pad] out
hipError_t launch_gather_fp8_rows(const void* q, const float* scales, const int32_t* map,
                                  int64_t T, int k, int H, void* q_perm, float* scales_perm,
                                  hipStream_t s, int groups = 0, int64_t R_pad = 0);
// Blockwise FP8 rows: codes [rows, H] and one scale per row and group of 128
// elements, stored group-major: scales[g * ld + r] (ld >= rows).
hipError_t launch_quantize_fp8_groups(const void* x, int64_t rows, int H,
                                      const int32_t* row_count, void* q, float* scales,
                                      int64_t ld, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v0, int32_t step, hipStream_t s);
hipError_t launch_fill_u16(uint16_t* p, int64_t n, uint16_t v, hipStream_t s);

int device_cu_count();

// Raises func's dynamic-LDS limit to `bytes` once per device; `done` holds
// the caller's per-device flags (a race between threads only repeats the
// call).
constexpr int kMaxDevices = 64;
inline hipError_t ensure_dynamic_lds(const void* func, int bytes, bool (&done)[kMaxDevices]) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool tracked = dev >= 0 && dev < kMaxDevices;
  if (tracked && done[dev]) return hipSuccess;
  e = hipFuncSetAttribute(func, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && tracked) done[dev] = true;
  return e;
}

}  // namespace moe
