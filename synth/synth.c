/*
 * Seeded synthetic inputs for the fused MoE layer.
 *
 * This module is shared by the CPU oracle's tests and by the GPU path's tests
 * and benchmark.  It holds no MoE arithmetic: it only draws numbers and packs
 * them into the storage formats the layer consumes (bf16, fp32, MXFP4).
 *
 * Generator: counter based, so every element is a pure function of
 * (seed, tensor_id, element_index) and the result does not depend on thread
 * count or order.
 *   - SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom
 *     number generators", OOPSLA 2014; constants as published by S. Vigna)
 *     hashes the counter into 64 random bits.
 *   - Box-Muller (G. Box, M. Muller, 1958) turns the uniforms of counters 2p
 *     and 2p+1 into the normals of elements 2p (cosine) and 2p+1 (sine).
 *
 * MXFP4 encoder (input construction only; the format is the OCP Microscaling
 * v1.0 one: e2m1 elements, one E8M0 scale per 32 elements along K):
 *   shared exponent e = floor(log2(amax)) - 2 (2 = emax of e2m1),
 *   scale byte = e + 127 clamped to [1, 254],
 *   element = round-to-nearest-even onto the e2m1 grid, saturating at 6.
 * Packing: byte j of a row holds element 2j in its low nibble and element
 * 2j+1 in its high nibble.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t sm64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tensor_id) {
  return sm64(sm64(seed) ^ (tensor_id * 0xD1B54A32D192ED03ull + 0x8CB92BA72F3D8DD7ull));
}

/* Standard normals 2p and 2p+1 of the stream with the given key: one
 * Box-Muller pair (cosine branch for the even index, sine for the odd). */
static inline void normal_pair(uint64_t key, uint64_t p, double* z0, double* z1) {
  uint64_t r1 = sm64(key + 2 * p);
  uint64_t r2 = sm64(key + 2 * p + 1);
  /* single precision is plenty for test data: u1 in (0, 1] on a 2^-24 grid */
  float u1 = (float)((r1 >> 40) + 1) * (1.0f / 16777216.0f);
  float u2 = (float)(r2 >> 40) * (1.0f / 16777216.0f);
  float r = sqrtf(-2.0f * logf(u1));
  float th = 6.2831853071795864769f * u2;
  *z0 = (double)(r * cosf(th));
  *z1 = (double)(r * sinf(th));
}

/* Standard normal number i of the stream with the given key. */
static inline double normal_at(uint64_t key, uint64_t i) {
  double z0, z1;
  normal_pair(key, i >> 1, &z0, &z1);
  return (i & 1) ? z1 : z0;
}

static inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* The SplitMix64 output function applied to state x (state already advanced). */
uint64_t synth_splitmix64(uint64_t x) { return sm64(x); }

uint64_t synth_raw_u64(uint64_t seed, uint64_t tensor_id, uint64_t i) {
  return sm64(stream_key(seed, tensor_id) + i);
}

double synth_normal_at(uint64_t seed, uint64_t tensor_id, uint64_t i) {
  return normal_at(stream_key(seed, tensor_id), i);
}

/* out[i] = (float)(mean + std * N_i) for i in [0, n); N_i from (seed, tensor_id). */
void synth_normal_f32(uint64_t seed, uint64_t tensor_id, int64_t n, double mean, double std,
                      float* out) {
  const uint64_t key = stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < (n + 1) / 2; ++p) {
    double z0, z1;
    normal_pair(key, (uint64_t)p, &z0, &z1);
    out[2 * p] = (float)(mean + std * z0);
    if (2 * p + 1 < n) out[2 * p + 1] = (float)(mean + std * z1);
  }
}

/* Same draw as synth_normal_f32, then rounded to bf16 (nearest, ties to even). */
void synth_normal_bf16(uint64_t seed, uint64_t tensor_id, int64_t n, double mean, double std,
                       uint16_t* out) {
  const uint64_t key = stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < (n + 1) / 2; ++p) {
    double z0, z1;
    normal_pair(key, (uint64_t)p, &z0, &z1);
    out[2 * p] = f32_to_bf16((float)(mean + std * z0));
    if (2 * p + 1 < n) out[2 * p + 1] = f32_to_bf16((float)(mean + std * z1));
  }
}

/* Row-biased fp32 logits: out[t*E+e] = (float)(N_{t*E+e} + bias[e]). */
void synth_biased_logits(uint64_t seed, uint64_t tensor_id, int64_t T, int64_t E,
                         const double* bias, float* out) {
  const uint64_t key = stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < T * E; ++i)
    out[i] = (float)(normal_at(key, (uint64_t)i) + bias[i % E]);
}

/* e2m1 magnitudes, code 0..7. */
static const float kE2M1Mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

static inline uint8_t e2m1_encode(float q) {
  uint8_t sign = (q < 0.0f) ? 8 : 0;
  float a = fabsf(q);
  if (!(a < 6.0f)) return (uint8_t)(sign | 7); /* saturate (also catches NaN input) */
  int best = 0;
  float bestd = a;
  for (int c = 1; c < 8; ++c) {
    float d = fabsf(a - kE2M1Mag[c]);
    /* strictly closer wins; on a tie the even code (mantissa bit 0) wins */
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      best = c;
      bestd = d;
    }
  }
  if (best == 0) return 0;
  return (uint8_t)(sign | best);
}

/* Quantize bf16 rows [rows, K] to MXFP4: packed [rows, K/2] and scales [rows, K/32].
 * K must be a multiple of 32. */
void synth_mxfp4_quantize(const uint16_t* w, int64_t rows, int64_t K, uint8_t* packed,
                          uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < K / 32; ++b) {
      const uint16_t* blk = w + r * K + b * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) {
        float v = fabsf(bf16_to_f32(blk[i]));
        if (v > amax) amax = v;
      }
      int e = 0;
      if (amax > 0.0f) e = (int)floor(log2((double)amax)) - 2;
      int sb = e + 127;
      if (sb < 1) sb = 1;
      if (sb > 254) sb = 254;
      e = sb - 127;
      scales[r * (K / 32) + b] = (uint8_t)sb;
      for (int i = 0; i < 32; i += 2) {
        float q0 = (float)ldexp((double)bf16_to_f32(blk[i]), -e);
        float q1 = (float)ldexp((double)bf16_to_f32(blk[i + 1]), -e);
        packed[r * (K / 2) + b * 16 + i / 2] =
            (uint8_t)(e2m1_encode(q0) | (e2m1_encode(q1) << 4));
      }
    }
  }
}
