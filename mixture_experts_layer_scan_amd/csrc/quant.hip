// FP8 E4M3 activations: the quantization step of [Quantize-Dispatch]
// (prepare() of vLLM's modular fused-MoE kernel quantizes the activations of
// the first GEMM; a2_scale makes the second GEMM's quantization consistent).
//
// Per row (one token, or one permuted row of the hidden activations):
//   dynamic:  a = max |x| over the row (448 for an all-zero row),
//             inv = 448 / a, scale = a / 448          (fp32, IEEE division)
//   static:   scale = *static_scale, inv = 1 / scale
//   q[j] = e4m3(clamp(x[j] * inv, -448, 448)),  x ~ q * scale
// The code is the OCP E4M3 value nearest to the clamped product, ties to the
// even code, computed with integer operations on the float's bits (so it does
// not depend on the conversion instructions' saturation rules).  With row
// multipliers (the routing weight applied to the input, top_k 1) the row is
// bf16(m * x) before quantization.  The quantized rows are then dispatched
// like bf16 rows: token-major, 16 bytes at a time, with their scales.
//
// Two terms (bf16 activations for the FP8 x e2m1 matrix cores): with
// v = clamp(x[j] * inv) as above, q1 = e4m3(v), the residual d = v - q1 (exact
// in fp32: v and q1 are within a factor of two, or d is a multiple of v's
// ulp below 2^-10) and q2 = e4m3(16 d), so x ~ scale * (q1 + q2 / 16) with
// about bf16's precision.  The row holds, per 64 k, the 64 codes of q1 and
// then the 64 codes of q2.
#include "moe_common.h"

#include <algorithm>

namespace moe {
namespace {

constexpr int kQuantThreads = 256;

// OCP E4M3 code of |v| <= 448 (finite), round to nearest even.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a < 0x3C800000u) {  // below 2^-6: multiples of 2^-9, the code is the count
    const float q = __builtin_rintf(__uint_as_float(a) * 512.0f);
    return sign | static_cast<uint32_t>(q);
  }
  // keep 3 mantissa bits: round at bit 20 to nearest even (a carry moves into
  // the exponent); the exponent is re-biased from 127 to 7
  const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
  return sign | (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
}

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// The value of an E4M3 code (exact in fp32).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e == 0 ? static_cast<float>(m) * 0.001953125f  // 2^-9
                           : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

// The 8 values of a 16-byte bf16 chunk, times m rounded back to bf16 when
// a row multiplier is given.
__device__ __forceinline__ void chunk_values(uint4 c, const float* mult, float m, float* v) {
  const uint32_t p[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(static_cast<uint16_t>(p[i] & 0xFFFFu));
    v[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(p[i] >> 16));
  }
  if (mult) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = bf16_to_f32(f32_to_bf16(m * v[i]));
  }
}

__global__ __launch_bounds__(kQuantThreads) void quantize_fp8_rows_kernel(
    const uint4* __restrict__ x, int64_t rows, int H8, const float* __restrict__ static_scale,
    const float* __restrict__ mult, const int32_t* __restrict__ row_count,
    uint2* __restrict__ q, float* __restrict__ scales, int terms) {
  __shared__ float s_max[kQuantThreads / kWave];
  const int64_t n = row_count ? static_cast<int64_t>(*row_count) : rows;
  const int lane = lane_id(), w = threadIdx.x / kWave;
  for (int64_t r = blockIdx.x; r < n && r < rows; r += gridDim.x) {
    const uint4* xr = x + r * H8;
    const float m = mult ? mult[r] : 1.0f;
    float inv, sc;
    if (static_scale) {
      sc = *static_scale;
      inv = 1.0f / sc;
    } else {
      float amax = 0.0f;
      for (int c = threadIdx.x; c < H8; c += blockDim.x) {
        float v[8];
        chunk_values(xr[c], mult, m, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
      }
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
      __syncthreads();  // the previous row's maxima are no longer read
      if (lane == 0) s_max[w] = amax;
      __syncthreads();
      amax = s_max[0];
      for (int i = 1; i < static_cast<int>(blockDim.x) / kWave; ++i) amax = fmaxf(amax, s_max[i]);
      if (amax == 0.0f) amax = 448.0f;
      inv = 448.0f / amax;
      sc = amax / 448.0f;
    }
    for (int c = threadIdx.x; c < H8; c += blockDim.x) {
      float v[8];
      chunk_values(xr[c], mult, m, v);
      if (terms == 2) {
        uint32_t c1[2] = {0, 0}, c2[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float a = clamp448(v[i] * inv);
          const uint32_t q1 = e4m3_rne(a);
          const uint32_t q2 = e4m3_rne((a - e4m3_value(q1)) * 16.0f);
          c1[i >> 2] |= q1 << (8 * (i & 3));
          c2[i >> 2] |= q2 << (8 * (i & 3));
        }
        // chunk c (k = 8c .. 8c + 7) of 64-k block c / 8
        uint2* qr = q + r * 2 * H8 + (c >> 3) * 16 + (c & 7);
        qr[0] = uint2{c1[0], c1[1]};
        qr[8] = uint2{c2[0], c2[1]};
        continue;
      }
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= e4m3_rne(clamp448(v[i] * inv)) << (8 * i);
        hi |= e4m3_rne(clamp448(v[4 + i] * inv)) << (8 * i);
      }
      q[r * H8 + c] = uint2{lo, hi};
    }
    if (threadIdx.x == 0) scales[r] = sc;
  }
}

// Blockwise FP8 (one scale per row and group of 128 consecutive elements,
// the per-token activation groups of block-scaled FP8): the per-row rule
// above applied to each group alone.  16 lanes take a group, 8 elements
// (one 16-byte chunk) each, so a wave quantizes 4 groups at once; the group
// maximum is a 16-lane reduction.  Scales are stored group-major,
// scales[g * ld + r] (the GEMM reads the scales of consecutive rows of one
// group together); rows at or past *row_count (when given) are skipped.
constexpr int kGroup = 128;

__global__ __launch_bounds__(kQuantThreads) void quantize_fp8_groups_kernel(
    const uint4* __restrict__ x, int64_t rows, int H8, const int32_t* __restrict__ row_count,
    uint2* __restrict__ q, float* __restrict__ scales, int64_t ld) {
  const int64_t n = row_count ? min(static_cast<int64_t>(*row_count), rows) : rows;
  const int groups = H8 / (kGroup / 8);
  const int lane = lane_id();
  const int sub = lane & 15;              // chunk of the group
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (blockDim.x / kWave);
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
  // group index gi = wave * 4 + lane / 16 (row-major over (row, group))
  for (int64_t gi0 = wave * 4; gi0 < n * groups; gi0 += waves * 4) {
    const int64_t gi = gi0 + (lane >> 4);
    const bool on = gi < n * groups;     // uniform per 16 lanes
    const int64_t r = on ? gi / groups : 0;
    const int g = on ? static_cast<int>(gi - r * groups) : 0;
    const int64_t c = r * H8 + g * (kGroup / 8) + sub;
    float v[8];
    chunk_values(on ? x[c] : uint4{0, 0, 0, 0}, nullptr, 1.0f, v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
    if (amax == 0.0f) amax = 448.0f;
    const float inv = 448.0f / amax;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= e4m3_rne(clamp448(v[i] * inv)) << (8 * i);
      hi |= e4m3_rne(clamp448(v[4 + i] * inv)) << (8 * i);
    }
    if (on) {
      q[c] = uint2{lo, hi};
      if (sub == 0) scales[g * ld + r] = amax / 448.0f;
    }
  }
}

// Dispatch of quantized rows: q_perm[map[t, j]] = q[t] (16 bytes at a time),
// scales_perm[map[t, j]] = scales[t].
__global__ __launch_bounds__(256) void gather_fp8_rows_kernel(const uint4* __restrict__ q,
                                                              const float* __restrict__ scales,
                                                              const int32_t* __restrict__ map,
                                                              int64_t T, int k, int H16,
                                                              uint4* __restrict__ q_perm,
                                                              float* __restrict__ scales_perm,
                                                              int groups, int64_t ld_src,
                                                              int64_t ld_dst) {
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const int32_t* mt = map + t * k;
    const uint4* src = q + t * H16;
    for (int c = threadIdx.x; c < H16; c += blockDim.x) {
      const uint4 v = src[c];
      for (int j = 0; j < k; ++j) {
        const int32_t r = mt[j];
        if (r >= 0) q_perm[static_cast<int64_t>(r) * H16 + c] = v;
      }
    }
    if (groups == 0) {
      if (threadIdx.x < k) {
        const int32_t r = mt[threadIdx.x];
        if (r >= 0) scales_perm[r] = scales[t];
      }
    } else {
      // group-major scales: scales_perm[g * ld_dst + r] = scales[g * ld_src + t]
      for (int i = threadIdx.x; i < k * groups; i += blockDim.x) {
        const int j = i / groups, g = i - j * groups;
        const int32_t r = mt[j];
        if (r >= 0) scales_perm[g * ld_dst + r] = scales[g * ld_src + t];
      }
    }
  }
}

}  // namespace

hipError_t launch_quantize_fp8(const void* x, int64_t rows, int H, const float* static_scale,
                               const float* mult, const int32_t* row_count, void* q,
                               float* scales, hipStream_t s, int terms) {
  if (rows <= 0) return hipSuccess;
  const int64_t blocks = rows < 16384 ? rows : 16384;
  hipLaunchKernelGGL(quantize_fp8_rows_kernel, dim3(static_cast<unsigned>(blocks)),
                     dim3(kQuantThreads), 0, s, static_cast<const uint4*>(x), rows, H / 8,
                     static_scale, mult, row_count, static_cast<uint2*>(q), scales, terms);
  return hipGetLastError();
}

hipError_t launch_gather_fp8_rows(const void* q, const float* scales, const int32_t* map,
                                  int64_t T, int k, int H, void* q_perm, float* scales_perm,
                                  hipStream_t s, int groups, int64_t R_pad) {
  if (T <= 0) return hipSuccess;
  const int64_t blocks = T < 8192 ? T : 8192;
  hipLaunchKernelGGL(gather_fp8_rows_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     s, static_cast<const uint4*>(q), scales, map, T, k, H / 16,
                     static_cast<uint4*>(q_perm), scales_perm, groups, T, R_pad);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8_groups(const void* x, int64_t rows, int H,
                                      const int32_t* row_count, void* q, float* scales,
                                      int64_t ld, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t groups = rows * (H / kGroup);
  const int64_t waves = (groups + 3) / 4;
  const int64_t blocks = std::min<int64_t>((waves + 3) / 4, 8192);
  hipLaunchKernelGGL(quantize_fp8_groups_kernel, dim3(static_cast<unsigned>(blocks)),
                     dim3(kQuantThreads), 0, s, static_cast<const uint4*>(x), rows, H / 8,
                     row_count, static_cast<uint2*>(q), scales, ld);
  return hipGetLastError();
}

}  // namespace moe
