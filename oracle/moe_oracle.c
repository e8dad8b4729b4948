/*
 * CPU oracle for the fused MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code with the HIP library.
 *
 * Plain, slow, obviously correct: per token, per routed expert, a dense
 * SiLU-gated MLP, all in double precision.  Every function names the passage
 * of the pages it follows.  Pages:
 *   [OUT]  vLLM "moe_output.py", module docstring (what a MoE layer returns
 *          when the code after it finishes the reduction): UnfinalizedMoEOutput,
 *          MoEOutput.
 *   [MOD]  vLLM "modular_kernel.py" (modular fused-MoE kernel): the stage
 *          comment [Router] -> [Quantize-Dispatch] -> [Permute-Experts-
 *          Unpermute] -> [Combine]; _moe_problem_size; prepare / finalize /
 *          apply / activation; FusedMoEModularKernel.forward.
 *   [EP]   vLLM "flashinfer_moe_ep.py": _E2M1_LUT, _dequant_fp4_ue8m0_gran32.
 *
 * Readings where the pages are silent:
 *   - w1 is [E, 2I, H]: rows [0, I) are the gate (SiLU'd), rows [I, 2I) the
 *     up projection; w2 is [E, H, I]; both contiguous along the reduction dim.
 *   - top-k is taken on the fp32 logits, ordered by logit descending, ties to
 *     the smaller expert id.
 *   - Routes of one local expert are placed in ascending expanded index
 *     t*k+j; experts in ascending local id; offsets are not padded.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_SOFTMAX = 0, OR_SIGMOID = 1 };
enum { OR_W_BF16 = 0, OR_W_MXFP4 = 1, OR_W_FP8 = 2, OR_W_FP8_BLOCK = 3 };
/* rows and columns of a weight block, elements of an activation group (block FP8) */
enum { OR_BLOCK = 128 };
enum { OR_ACT_SILU = 0, OR_ACT_GELU = 1 };

typedef struct {
  int32_t fmt;            /* OR_W_BF16, OR_W_MXFP4, OR_W_FP8 or OR_W_FP8_BLOCK */
  const void* data;       /* bf16 [rows, K], packed e2m1 [rows, K/2] or e4m3 [rows, K] */
  const void* scales;     /* E8M0 u8 [rows, K/32] (MXFP4), fp32 [rows] (FP8, per row) or
                             fp32 [rows/128, K/128] (FP8_BLOCK, per 128 x 128 block) */
} oracle_weights;

static double bf16_val(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* float -> bf16 bits, round to nearest even (finite inputs). */
static uint16_t bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* ---- MXFP4 decode ([EP] _E2M1_LUT and _dequant_fp4_ue8m0_gran32) ----------
 * e2m1 code -> value table as the page prints it (code 8 is -0.0).  The scale
 * byte s is read as the float whose bit pattern is s<<23: 2^(s-127) for
 * 1 <= s <= 254, +0.0 for s = 0 and +inf for s = 255. */
static const double kE2M1[16] = {0.0,  0.5,  1.0,  1.5,  2.0,  3.0,  4.0,  6.0,
                                 -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0};

double oracle_e8m0_scale(uint8_t s) {
  if (s == 0) return 0.0;
  if (s == 255) return INFINITY;
  return ldexp(1.0, (int)s - 127);
}

/* Element kk of packed row `row` (K elements per row): low nibble = even kk. */
double oracle_mxfp4_value(const uint8_t* packed, const uint8_t* scales, int64_t row, int64_t K,
                          int64_t kk) {
  uint8_t b = packed[row * (K / 2) + kk / 2];
  uint8_t code = (kk & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 0x0F);
  return kE2M1[code] * oracle_e8m0_scale(scales[row * (K / 32) + kk / 32]);
}

/* ---- FP8 E4M3 (the OCP 8-bit float with 4 exponent bits, bias 7, 3 mantissa
 * bits, no infinities, S.1111.111 = NaN; largest finite 448): the FP8 type of
 * the quantized activations of [MOD] prepare / apply (quant_dtype, a1_scale,
 * a2_scale, w1_scale, w2_scale; the pages name no layout, this one is the
 * MI355X matrix cores') --------------------------------------------------------
 * decode: exponent field e, mantissa m: e = 0 -> m * 2^-9; else
 * (1 + m/8) * 2^(e-7). */
double oracle_e4m3_decode(uint8_t c) {
  int e = (c >> 3) & 15, m = c & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  mag = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return (c & 0x80) ? -mag : mag;
}

/* encode: the nearest e4m3 value, ties to the even code; |v| >= 448 gives
 * +-448 (saturation; the quantizers below never pass more). */
uint8_t oracle_e4m3_encode(double v) {
  uint8_t sign = (v < 0.0 || (v == 0.0 && signbit(v))) ? 0x80 : 0;
  double a = fabs(v);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  if (a < ldexp(1.0, -6)) {  /* subnormal range: steps of 2^-9, code = steps */
    double q = nearbyint(a / ldexp(1.0, -9));  /* ties to even */
    return (uint8_t)(sign | (uint8_t)q);        /* q = 8 is the smallest normal */
  }
  int ex;
  frexp(a, &ex);               /* a = f * 2^ex, f in [0.5, 1) */
  int e = ex - 1;              /* a in [2^e, 2^(e+1)) */
  double q = nearbyint(a / ldexp(1.0, e - 3));  /* 8 .. 16, ties to even */
  if (q == 16.0) { q = 8.0; e += 1; }
  return (uint8_t)(sign | (uint8_t)((e + 7) << 3) | (uint8_t)(q - 8.0));
}

/* Per-row FP8 quantization of bf16 rows (the per-token activation quantization
 * of prepare, per_act_token_quant; a static a1_scale / a2_scale otherwise).
 * In float32, as the quantizing kernel decides the codes:
 *   dynamic: a = max |x| over the row (448 when the row is all zero),
 *            inv = 448 / a, scale = a / 448;
 *   static:  scale = *static_scale, inv = 1 / scale;
 *   q[j] = e4m3(min(max(x[j] * inv, -448), 448)), and x ~ q * scale. */
void oracle_quantize_fp8_rows(const uint16_t* x, int64_t rows, int64_t H,
                              const float* static_scale, uint8_t* q, float* scales) {
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t* xr = x + r * H;
    float inv, sc;
    if (static_scale) {
      sc = *static_scale;
      inv = 1.0f / sc;
    } else {
      float amax = 0.0f;
      for (int64_t j = 0; j < H; ++j) {
        float a = fabsf((float)bf16_val(xr[j]));
        if (a > amax) amax = a;
      }
      if (amax == 0.0f) amax = 448.0f;
      inv = 448.0f / amax;
      sc = amax / 448.0f;
    }
    for (int64_t j = 0; j < H; ++j) {
      float v = (float)bf16_val(xr[j]) * inv;
      if (v > 448.0f) v = 448.0f;
      if (v < -448.0f) v = -448.0f;
      q[r * H + j] = oracle_e4m3_encode((double)v);
    }
    scales[r] = sc;
  }
}

/* Two-term FP8 quantization of bf16 rows: bf16 activations carried to the
 * FP8 x e2m1 matrix cores at close to bf16 precision (the quantize step of
 * prepare for MXFP4 weights).  Per row, with the dynamic scale and inv of
 * oracle_quantize_fp8_rows, in float32 as the kernel decides the codes:
 *   v = min(max(x[j] * inv, -448), 448),  q1[j] = e4m3(v),
 *   d = v - value(q1[j])                  (a difference of two nearby
 *                                          floats: exact),
 *   q2[j] = e4m3(16 d),
 * so x[j] ~ scale * (value(q1) + value(q2) / 16). */
void oracle_quantize_fp8x2_rows(const uint16_t* x, int64_t rows, int64_t H, uint8_t* q1,
                                uint8_t* q2, float* scales) {
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t* xr = x + r * H;
    float amax = 0.0f;
    for (int64_t j = 0; j < H; ++j) {
      float a = fabsf((float)bf16_val(xr[j]));
      if (a > amax) amax = a;
    }
    if (amax == 0.0f) amax = 448.0f;
    const float inv = 448.0f / amax;
    for (int64_t j = 0; j < H; ++j) {
      float v = (float)bf16_val(xr[j]) * inv;
      if (v > 448.0f) v = 448.0f;
      if (v < -448.0f) v = -448.0f;
      const uint8_t c1 = oracle_e4m3_encode((double)v);
      const double d = (double)v - oracle_e4m3_decode(c1);
      q1[r * H + j] = c1;
      q2[r * H + j] = oracle_e4m3_encode(16.0 * d);
    }
    scales[r] = amax / 448.0f;
  }
}

/* Block-scaled FP8 activations ([MOD] FusedMoEPermuteExpertsUnpermute quant
 * properties: block_shape, with per_act_token_quant the activations scaled
 * per token; the page names the knobs, not the rule): every group of G
 * consecutive elements of a row gets its own scale, by the per-row rule of
 * oracle_quantize_fp8_rows applied to the group alone.  scales is
 * [rows, H / G]. */
void oracle_quantize_fp8_groups(const uint16_t* x, int64_t rows, int64_t H, int64_t G, uint8_t* q,
                                float* scales) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t g = 0; g < H / G; ++g)
      oracle_quantize_fp8_rows(x + r * H + g * G, 1, G, NULL, q + r * H + g * G,
                               scales + r * (H / G) + g);
}

/* A row quantized by oracle_quantize_fp8_rows (terms 1) or
 * oracle_quantize_fp8x2_rows (terms 2), decoded to doubles. */
static void quantize_decode(const uint16_t* row, int64_t n, int terms, const float* static_scale,
                            uint8_t* c1, uint8_t* c2, double* out) {
  float sc;
  if (terms == 3) {  /* block FP8: one scale per 128 elements */
    float gs[1024];
    oracle_quantize_fp8_groups(row, 1, n, OR_BLOCK, c1, gs);
    for (int64_t c = 0; c < n; ++c)
      out[c] = oracle_e4m3_decode(c1[c]) * (double)gs[c / OR_BLOCK];
    return;
  }
  if (terms == 2) {
    oracle_quantize_fp8x2_rows(row, 1, n, c1, c2, &sc);
    for (int64_t c = 0; c < n; ++c)
      out[c] = (oracle_e4m3_decode(c1[c]) + oracle_e4m3_decode(c2[c]) / 16.0) * (double)sc;
  } else {
    oracle_quantize_fp8_rows(row, 1, n, static_scale, c1, &sc);
    for (int64_t c = 0; c < n; ++c) out[c] = oracle_e4m3_decode(c1[c]) * (double)sc;
  }
}

/* Weight element (row, kk) of a [rows, K] matrix in any storage format (FP8:
 * the code times the row's scale, per_out_ch_quant). */
double oracle_weight_at(const oracle_weights* w, int64_t row, int64_t K, int64_t kk) {
  if (w->fmt == OR_W_MXFP4)
    return oracle_mxfp4_value((const uint8_t*)w->data, (const uint8_t*)w->scales, row, K, kk);
  if (w->fmt == OR_W_FP8)
    return oracle_e4m3_decode(((const uint8_t*)w->data)[row * K + kk]) *
           (double)((const float*)w->scales)[row];
  if (w->fmt == OR_W_FP8_BLOCK)
    return oracle_e4m3_decode(((const uint8_t*)w->data)[row * K + kk]) *
           (double)((const float*)w->scales)[(row / OR_BLOCK) * (K / OR_BLOCK) + kk / OR_BLOCK];
  return bf16_val(((const uint16_t*)w->data)[row * K + kk]);
}

/* sum_kk W[row, kk] * v[kk], ascending kk, in double. */
static double dot_row(const oracle_weights* w, int64_t row, int64_t K, const double* v) {
  double acc = 0.0;
  if (w->fmt == OR_W_MXFP4) {
    const uint8_t* p = (const uint8_t*)w->data + row * (K / 2);
    const uint8_t* s = (const uint8_t*)w->scales + row * (K / 32);
    /* the scale of each 32-element block, decoded once per block */
    for (int64_t b0 = 0; b0 < K; b0 += 32) {
      const double sc = oracle_e8m0_scale(s[b0 / 32]);
      for (int64_t kk = b0; kk < b0 + 32; ++kk) {
        uint8_t b = p[kk / 2];
        uint8_t code = (kk & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 0x0F);
        acc += kE2M1[code] * sc * v[kk];
      }
    }
  } else if (w->fmt == OR_W_FP8) {
    /* the 256 decoded values, each from oracle_e4m3_decode */
    static double table[256];
    static int ready = 0;
#pragma omp critical(e4m3_table)
    if (!ready) {
      for (int c = 0; c < 256; ++c) table[c] = oracle_e4m3_decode((uint8_t)c);
      ready = 1;
    }
    const uint8_t* p = (const uint8_t*)w->data + row * K;
    const double sc = (double)((const float*)w->scales)[row];
    for (int64_t kk = 0; kk < K; ++kk) acc += table[p[kk]] * sc * v[kk];
  } else if (w->fmt == OR_W_FP8_BLOCK) {
    /* element (row, kk) = code * the scale of its 128 x 128 block */
    const uint8_t* p = (const uint8_t*)w->data + row * K;
    const float* s = (const float*)w->scales + (row / OR_BLOCK) * (K / OR_BLOCK);
    for (int64_t kk = 0; kk < K; ++kk)
      acc += oracle_e4m3_decode(p[kk]) * (double)s[kk / OR_BLOCK] * v[kk];
  } else {
    const uint16_t* p = (const uint16_t*)w->data + row * K;
    for (int64_t kk = 0; kk < K; ++kk) acc += bf16_val(p[kk]) * v[kk];
  }
  return acc;
}

/* ---- [Router] ([MOD] stage comment; [OUT] expert_weights carry the routed
 * scaling factor when the routing method folds it in) ------------------------
 * For token t: pick k experts by repeatedly taking the largest remaining
 * logit (scan in ascending id, strict '>' so ties keep the smaller id).
 * Scores: softmax over all E experts, or the logistic sigmoid of each logit.
 * With renormalize the k selected scores are divided by their sum.  The
 * result is multiplied by rsf. */
void oracle_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t score_fn,
                  int32_t renormalize, double rsf, int32_t* ids, double* weights) {
  char* taken = (char*)malloc((size_t)E);
  double* score = (double*)malloc(sizeof(double) * (size_t)E);
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
      taken[best] = 1;
      ids[t * k + j] = best;
    }
    if (score_fn == OR_SOFTMAX) {
      double m = l[0];
      for (int e = 1; e < E; ++e)
        if (l[e] > m) m = l[e];
      double z = 0.0;
      for (int e = 0; e < E; ++e) z += exp((double)l[e] - m);
      for (int e = 0; e < E; ++e) score[e] = exp((double)l[e] - m) / z;
    } else {
      for (int e = 0; e < E; ++e) score[e] = 1.0 / (1.0 + exp(-(double)l[e]));
    }
    double sel = 0.0;
    for (int j = 0; j < k; ++j) sel += score[ids[t * k + j]];
    for (int j = 0; j < k; ++j) {
      double w = score[ids[t * k + j]];
      if (renormalize) w /= sel;
      weights[t * k + j] = w * rsf;
    }
  }
  free(taken);
  free(score);
}

/* ---- Permute ([MOD] prepare: expert_map maps global to local expert ids and
 * the per-local-expert token counts; [OUT] expanded_idx_to_permuted_idx is
 * int32 [num_tokens, top_k] with -1 for an expert that is not local) --------
 * L = expert_map[id] (or id when there is no map).  counts[L] = routes to L;
 * offsets = exclusive prefix sum of counts (E_l + 1 entries).  Walking the
 * expanded index x = t*k + j upward, map[x] = offsets[L] + (routes to L seen
 * so far), or -1 when L < 0.  Returns 0, or -1 on an id outside [0, E) or a
 * local id outside [-1, E_l). */
int oracle_permute(const int32_t* ids, const int32_t* expert_map, int64_t T, int32_t k,
                   int32_t E, int32_t E_l, int32_t* map, int32_t* offsets, int32_t* counts) {
  int64_t R = T * k;
  for (int e = 0; e < E_l; ++e) counts[e] = 0;
  for (int64_t x = 0; x < R; ++x) {
    int32_t id = ids[x];
    if (id < 0 || id >= E) return -1;
    int32_t L = expert_map ? expert_map[id] : id;
    if (L < -1 || L >= E_l) return -1;
    if (L >= 0) counts[L] += 1;
  }
  offsets[0] = 0;
  for (int e = 0; e < E_l; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* seen = (int32_t*)calloc((size_t)(E_l > 0 ? E_l : 1), sizeof(int32_t));
  for (int64_t x = 0; x < R; ++x) {
    int32_t L = expert_map ? expert_map[ids[x]] : ids[x];
    if (L < 0) {
      map[x] = -1;
    } else {
      map[x] = offsets[L] + seen[L];
      seen[L] += 1;
    }
  }
  free(seen);
  return 0;
}

/* ---- Permute into the batched experts format ([MOD] FusedMoEActivationFormat
 * BatchedExperts: activations laid out as (local experts, max tokens per
 * expert, hidden); prepare returns the per-local-expert token counts with
 * them; _moe_problem_size reads M = max_num_tokens from that layout) ---------
 * Expert L's rows are [L * max_tokens, (L + 1) * max_tokens).  Walking the
 * expanded index x = t*k + j upward, the n-th route to L (n = 0, 1, ...) goes
 * to row L * max_tokens + n while n < max_tokens; a route past that capacity,
 * or to an expert that is not local, gets -1.  counts[L] = all routes to L
 * (it exceeds max_tokens exactly when routes were dropped).  Returns 0, or -1
 * on an id outside [0, E) or a local id outside [-1, E_l). */
int oracle_permute_batched(const int32_t* ids, const int32_t* expert_map, int64_t T, int32_t k,
                           int32_t E, int32_t E_l, int32_t max_tokens, int32_t* map,
                           int32_t* counts) {
  int64_t R = T * k;
  for (int e = 0; e < E_l; ++e) counts[e] = 0;
  for (int64_t x = 0; x < R; ++x) {
    int32_t id = ids[x];
    if (id < 0 || id >= E) return -1;
    int32_t L = expert_map ? expert_map[id] : id;
    if (L < -1 || L >= E_l) return -1;
    if (L < 0) {
      map[x] = -1;
      continue;
    }
    map[x] = counts[L] < max_tokens ? L * max_tokens + counts[L] : -1;
    counts[L] += 1;
  }
  return 0;
}

/* ---- Experts ([MOD] apply: GEMM1, activation, GEMM2, unweighted; activation:
 * the output is half the width of the input, "silu" gives
 * silu(first half) * second half and "gelu" gelu(first half) * second half;
 * _moe_problem_size: w1 is [E, N, .], w2 is [E, K, .] with K the hidden
 * size) ----------------------------------------------------------------------
 * h[i] = act(g_i) * u_i with g_i = W1[e, i, :] . x, u_i = W1[e, I + i, :] . x,
 *   silu(g) = g / (1 + exp(-g)),   gelu(g) = g/2 * (1 + erf(g / sqrt(2)))
 * (the erf form of GELU).  With clamp > 0 (the activation_clamp of the fused
 * SwiGLU epilogue in [EP] build_fi_mega_config; the page gives only its name
 * and type) the gate is limited from above and the up value to [-clamp,
 * clamp] before the product: g = min(g, clamp), u = min(max(u, -clamp), clamp). */
static double gated_act(double g, double u, int32_t act, double clamp) {
  if (clamp > 0.0) {
    if (g > clamp) g = clamp;
    if (u > clamp) u = clamp;
    if (u < -clamp) u = -clamp;
  }
  double a = act == OR_ACT_GELU ? 0.5 * g * (1.0 + erf(g / sqrt(2.0))) : g / (1.0 + exp(-g));
  return a * u;
}

void oracle_expert_hidden_act(const double* x, int64_t H, int64_t I, const oracle_weights* w1,
                              int64_t e, int32_t act, double clamp, double* h) {
  for (int64_t i = 0; i < I; ++i) {
    double g = dot_row(w1, e * 2 * I + i, H, x);
    double u = dot_row(w1, e * 2 * I + I + i, H, x);
    h[i] = gated_act(g, u, act, clamp);
  }
}

void oracle_expert_hidden(const double* x, int64_t H, int64_t I, const oracle_weights* w1,
                          int64_t e, double* h) {
  oracle_expert_hidden_act(x, H, I, w1, e, OR_ACT_SILU, 0.0, h);
}

/* y[n] = W2[e, n, :] . h */
void oracle_expert_out(const double* h, int64_t H, int64_t I, const oracle_weights* w2,
                       int64_t e, double* y) {
  for (int64_t n = 0; n < H; ++n) y[n] = dot_row(w2, e * H + n, I, h);
}

/* Batched helpers over bf16 rows (parallel over rows; each row is the plain
 * per-row function above).  Used to check the two grouped GEMMs on their own:
 *   hidden: rows[r] -> h[r] with expert expert_of_row[r];
 *   out:    h rows (bf16) -> y[r]. */
void oracle_hidden_rows(const uint16_t* a, int64_t rows, int64_t H, int64_t I,
                        const oracle_weights* w1, const int32_t* expert_of_row, int32_t act,
                        double clamp, double* h) {
#pragma omp parallel
  {
    double* xv = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
      for (int64_t c = 0; c < H; ++c) xv[c] = bf16_val(a[r * H + c]);
      oracle_expert_hidden_act(xv, H, I, w1, expert_of_row[r], act, clamp, h + r * I);
    }
    free(xv);
  }
}

/* The same on FP8 rows (codes [rows, K] and one scale per group of `group`
 * consecutive elements of a row: group = K for one scale per row, as
 * oracle_quantize_fp8_rows writes them, 128 for block-scaled rows as
 * oracle_quantize_fp8_groups writes them): the rows are decoded to
 * q * the scale of q's group. */
void oracle_hidden_rows_fp8(const uint8_t* aq, const float* a_scales, int64_t group, int64_t rows,
                            int64_t H, int64_t I, const oracle_weights* w1,
                            const int32_t* expert_of_row, int32_t act, double clamp, double* h) {
#pragma omp parallel
  {
    double* xv = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
      for (int64_t c = 0; c < H; ++c)
        xv[c] = oracle_e4m3_decode(aq[r * H + c]) * (double)a_scales[r * (H / group) + c / group];
      oracle_expert_hidden_act(xv, H, I, w1, expert_of_row[r], act, clamp, h + r * I);
    }
    free(xv);
  }
}

void oracle_out_rows_fp8(const uint8_t* hq, const float* h_scales, int64_t group, int64_t rows,
                         int64_t I, int64_t H, const oracle_weights* w2,
                         const int32_t* expert_of_row, double* y) {
#pragma omp parallel
  {
    double* hv = (double*)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
      for (int64_t c = 0; c < I; ++c)
        hv[c] = oracle_e4m3_decode(hq[r * I + c]) * (double)h_scales[r * (I / group) + c / group];
      oracle_expert_out(hv, H, I, w2, expert_of_row[r], y + r * H);
    }
    free(hv);
  }
}

/* The same on two-term FP8 rows (codes q1, q2 [rows, K] and one scale per
 * row, as oracle_quantize_fp8x2_rows writes them): the rows are decoded to
 * (q1 + q2 / 16) * scale. */
void oracle_hidden_rows_fp8x2(const uint8_t* q1, const uint8_t* q2, const float* a_scales,
                              int64_t rows, int64_t H, int64_t I, const oracle_weights* w1,
                              const int32_t* expert_of_row, int32_t act, double clamp,
                              double* h) {
#pragma omp parallel
  {
    double* xv = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
      for (int64_t c = 0; c < H; ++c)
        xv[c] = (oracle_e4m3_decode(q1[r * H + c]) + oracle_e4m3_decode(q2[r * H + c]) / 16.0) *
                (double)a_scales[r];
      oracle_expert_hidden_act(xv, H, I, w1, expert_of_row[r], act, clamp, h + r * I);
    }
    free(xv);
  }
}

void oracle_out_rows_fp8x2(const uint8_t* q1, const uint8_t* q2, const float* h_scales,
                           int64_t rows, int64_t I, int64_t H, const oracle_weights* w2,
                           const int32_t* expert_of_row, double* y) {
#pragma omp parallel
  {
    double* hv = (double*)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
      for (int64_t c = 0; c < I; ++c)
        hv[c] = (oracle_e4m3_decode(q1[r * I + c]) + oracle_e4m3_decode(q2[r * I + c]) / 16.0) *
                (double)h_scales[r];
      oracle_expert_out(hv, H, I, w2, expert_of_row[r], y + r * H);
    }
    free(hv);
  }
}

void oracle_out_rows(const uint16_t* hb, int64_t rows, int64_t I, int64_t H,
                     const oracle_weights* w2, const int32_t* expert_of_row, double* y) {
#pragma omp parallel
  {
    double* hv = (double*)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
      for (int64_t c = 0; c < I; ++c) hv[c] = bf16_val(hb[r * I + c]);
      oracle_expert_out(hv, H, I, w2, expert_of_row[r], y + r * H);
    }
    free(hv);
  }
}

/* ---- [Combine] ([MOD] finalize: apply the weights to the unweighted expert
 * output and reduce over top-k, written into an output that starts at zero
 * (forward allocates zeros_like); [OUT] MoEOutput: the routed scaling factor
 * multiplies the routed sum before the shared-expert add; -1 entries of the
 * map name no row) -----------------------------------------------------------
 * out[t] = rsf_fin * sum_{j : map[t,j] >= 0} w[t,j] * Y[map[t,j]] + shared[t]. */
void oracle_finalize(const uint16_t* y_perm, const double* w, const int32_t* map, int64_t T,
                     int32_t k, int64_t H, double rsf_fin, const uint16_t* shared, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* o = out + t * H;
    for (int64_t n = 0; n < H; ++n) o[n] = 0.0;
    for (int j = 0; j < k; ++j) {
      int32_t r = map[t * k + j];
      if (r < 0) continue;
      for (int64_t n = 0; n < H; ++n) o[n] += w[t * k + j] * bf16_val(y_perm[(int64_t)r * H + n]);
    }
    for (int64_t n = 0; n < H; ++n) {
      o[n] *= rsf_fin;
      if (shared) o[n] += bf16_val(shared[t * H + n]);
    }
  }
}

/* ---- Fused tail on one GPU ([OUT] MoEOutput docstring: the layer may leave
 * the top-k sum, the routed scaling factor and the shared add for the code
 * that follows it, usually the next layer's normalization, to carry out) -----
 * For each token t, with m[t] the finalize output above:
 *   residual_out[t] = residual[t] + m[t]
 *   out[t, n] = residual_out[t, n] / sqrt(mean_n residual_out[t, n]^2 + eps)
 *               * gamma[n]
 * (the RMSNorm of the new residual stream, scaled per column by gamma). */
void oracle_finalize_add_rmsnorm(const uint16_t* y_perm, const double* w, const int32_t* map,
                                 int64_t T, int32_t k, int64_t H, double rsf_fin,
                                 const uint16_t* shared, const uint16_t* residual,
                                 const uint16_t* gamma, double eps, double* residual_out,
                                 double* out) {
  oracle_finalize(y_perm, w, map, T, k, H, rsf_fin, shared, residual_out);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* r = residual_out + t * H;
    double ss = 0.0;
    for (int64_t n = 0; n < H; ++n) {
      r[n] += bf16_val(residual[t * H + n]);
      ss += r[n] * r[n];
    }
    const double inv = 1.0 / sqrt(ss / (double)H + eps);
    for (int64_t n = 0; n < H; ++n) out[t * H + n] = r[n] * inv * bf16_val(gamma[n]);
  }
}

/* ---- The whole layer on selected tokens ([MOD] forward: prepare, apply,
 * finalize; [OUT] MoEOutput for the shared add) -------------------------------
 * For each listed token t: route it, localize each route through the expert
 * map, run the expert MLP of every local route, and combine:
 *   out[t] = rsf_fin * sum_j w_j * MLP_{L_j}(x_t) + MLP_shared(x_t).
 * With weight_on_input ([MOD] forward and prepare: apply_router_weight_on_input
 * puts the weights on the activations before dispatch, and finalize then does
 * not apply them; only for top_k = 1):
 *   out[t] = rsf_fin * sum_j MLP_{L_j}(w_j * x_t) + MLP_shared(x_t).
 * act and clamp select the activation of every expert MLP, the shared one
 * included (see gated_act).
 * With act_quant (FP8 activations: [MOD] prepare quantizes a1 for the first
 * GEMM, a2_scale keeps the second GEMM's quantization consistent) each routed
 * expert sees its input row as bf16 (x, or bf16(w_j * x) with
 * weight_on_input) quantized per row to FP8 (oracle_quantize_fp8_rows; static
 * a1_scale when given), and its hidden row h rounded to bf16 and quantized
 * the same way (static a2_scale when given).  act_quant 2 quantizes both rows
 * with the two-term rule instead (oracle_quantize_fp8x2_rows, dynamic scales);
 * act_quant 3 (block-scaled FP8) quantizes them per group of 128 elements
 * (oracle_quantize_fp8_groups, dynamic scales).
 * The shared expert stays bf16.
 * Optional outputs: y_routes [n, k, H] (the unweighted per-route expert output,
 * zero for non-local routes), ids [n, k], weights [n, k].
 * shared_I = 0 disables the shared expert. */
void oracle_moe_tokens(const uint16_t* x, int64_t H, int64_t I, const float* logits, int32_t E,
                       int32_t k, int32_t score_fn, int32_t renormalize, double rsf,
                       const int32_t* expert_map, const oracle_weights* w1,
                       const oracle_weights* w2, int64_t shared_I, const uint16_t* ws1,
                       const uint16_t* ws2, double rsf_fin, int32_t act, double clamp,
                       int32_t weight_on_input, int32_t act_quant, const float* a1_scale,
                       const float* a2_scale, const int64_t* tokens, int64_t n_tokens,
                       double* out, double* y_routes, int32_t* ids_out, double* w_out) {
  oracle_weights s1 = {OR_W_BF16, ws1, NULL};
  oracle_weights s2 = {OR_W_BF16, ws2, NULL};
#pragma omp parallel
  {
    int64_t Imax = I > shared_I ? I : shared_I;
    double* xv = (double*)malloc(sizeof(double) * (size_t)H);
    double* xw = (double*)malloc(sizeof(double) * (size_t)H);
    double* hv = (double*)malloc(sizeof(double) * (size_t)Imax);
    double* yv = (double*)malloc(sizeof(double) * (size_t)H);
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    double* wts = (double*)malloc(sizeof(double) * (size_t)k);
    int64_t Qmax = H > I ? H : I;
    uint16_t* qin = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)Qmax);
    uint8_t* qout = (uint8_t*)malloc((size_t)Qmax);
    uint8_t* qout2 = (uint8_t*)malloc((size_t)Qmax);
#pragma omp for schedule(dynamic, 1)
    for (int64_t s = 0; s < n_tokens; ++s) {
      int64_t t = tokens[s];
      for (int64_t c = 0; c < H; ++c) xv[c] = bf16_val(x[t * H + c]);
      oracle_route(logits + t * E, 1, E, k, score_fn, renormalize, rsf, ids, wts);
      double* o = out + s * H;
      for (int64_t n = 0; n < H; ++n) o[n] = 0.0;
      for (int j = 0; j < k; ++j) {
        int32_t L = expert_map ? expert_map[ids[j]] : ids[j];
        if (ids_out) ids_out[s * k + j] = ids[j];
        if (w_out) w_out[s * k + j] = wts[j];
        double* yr = y_routes ? y_routes + (s * k + j) * H : yv;
        if (L < 0) {
          for (int64_t n = 0; n < H; ++n) yr[n] = 0.0;
          continue;
        }
        const double* xin = xv;
        if (weight_on_input) {
          for (int64_t c = 0; c < H; ++c) xw[c] = wts[j] * xv[c];
          xin = xw;
        }
        if (act_quant) {
          for (int64_t c = 0; c < H; ++c)
            qin[c] = weight_on_input ? bf16_bits((float)wts[j] * (float)xv[c]) : x[t * H + c];
          quantize_decode(qin, H, act_quant, a1_scale, qout, qout2, xw);
          xin = xw;
        }
        oracle_expert_hidden_act(xin, H, I, w1, L, act, clamp, hv);
        if (act_quant) {
          for (int64_t c = 0; c < I; ++c) qin[c] = bf16_bits((float)hv[c]);
          quantize_decode(qin, I, act_quant, a2_scale, qout, qout2, hv);
        }
        oracle_expert_out(hv, H, I, w2, L, yr);
        const double wj = weight_on_input ? 1.0 : wts[j];
        for (int64_t n = 0; n < H; ++n) o[n] += wj * yr[n];
      }
      for (int64_t n = 0; n < H; ++n) o[n] *= rsf_fin;
      if (shared_I > 0) {
        oracle_expert_hidden_act(xv, H, shared_I, &s1, 0, act, clamp, hv);
        oracle_expert_out(hv, H, shared_I, &s2, 0, yv);
        for (int64_t n = 0; n < H; ++n) o[n] += yv[n];
      }
    }
    free(xv);
    free(xw);
    free(hv);
    free(yv);
    free(ids);
    free(wts);
    free(qin);
    free(qout);
    free(qout2);
  }
}

int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
  return n;
}
