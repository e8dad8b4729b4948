/*
 * moe.h -- C ABI of the fused Mixture-of-Experts layer for AMD Instinct MI355X
 * (gfx950 / CDNA4).
 *
 * The layer follows the stage decomposition of vLLM's modular fused-MoE kernel
 * (page "modular_kernel.py", the module comment: Router -> Quantize-Dispatch
 * -> Permute-Experts-Unpermute -> Combine):
 *
 *   moe_route_topk         Router: top-k experts per token and their weights
 *   moe_permute            Quantize-Dispatch (single-GPU part): the permute map
 *                          and per-local-expert row offsets, and the gather of
 *                          token rows into expert-contiguous order
 *   moe_grouped_gemm1_act  Experts, GEMM1 with the SiLU(gate) * up activation
 *   moe_grouped_gemm2      Experts, GEMM2 (unweighted, unreduced output)
 *   moe_finalize           Unpermute + Combine: weights, top-k reduction,
 *                          optional shared-expert add
 *   moe_fused_experts_unfinalized
 *                          all but the last step; returns the three buffers of
 *                          the deferred-finalize contract (page "moe_output.py",
 *                          UnfinalizedMoEOutput)
 *   moe_fused_experts      the whole layer, finalized
 *
 * Conventions for every call
 *   - Memory: the caller owns every buffer.  Pointers marked (device) must be
 *     device memory of the current HIP device; nothing is allocated, freed or
 *     copied between host and device by these calls, and the host never waits
 *     for the device.  Work is enqueued on `stream` (a hipStream_t; NULL is the
 *     null stream), so every call can be captured into a HIP graph.
 *   - Layout: arrays are dense and row-major with the shapes given, with no
 *     padding between rows; bf16 arrays hold IEEE bfloat16 bit patterns.
 *     Device pointers must be 16-byte aligned.
 *   - Sizes are explicit arguments.  Nothing is inferred from a trailing
 *     dimension, since packed 4-bit weights halve it (page "modular_kernel.py",
 *     _moe_problem_size).
 *   - Names: T tokens, H hidden size, I expert intermediate size, E global
 *     experts, E_l local experts, k top_k, R = T*k routes, R_l routes to local
 *     experts, R_pad >= R the row count of permuted buffers.
 *   - Errors: each call returns MOE_OK (0) or a negative moe_status and
 *     enqueues nothing when it fails; moe_last_error() gives a thread-local
 *     message.  T = 0 is valid and enqueues nothing.
 *   - Calls on one stream run in order; two calls that write the same buffer
 *     on different streams race.
 */
#ifndef MOE_MI355X_MOE_H_
#define MOE_MI355X_MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  They mirror the checks of the output-contract page
 * (convert_flashinfer_moe_output raises ValueError on: negative num_tokens,
 * non-positive top_k, a deferred output given a destination, a non-int32 map,
 * element counts other than num_tokens * top_k, mixed devices, non-contiguous
 * buffers). */
typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = -1,     /* T < 0, k <= 0, k > E, E_l > E, bad size  */
  MOE_ERR_UNSUPPORTED = -2,          /* dtype, score function or activation tag  */
  MOE_ERR_SIZE_MISMATCH = -3,        /* R_pad < T*k, workspace too small         */
  MOE_ERR_MISALIGNED = -4,           /* a device pointer not 16-byte aligned     */
  MOE_ERR_DEVICE = -5,               /* a pointer that is not device memory      */
  MOE_ERR_DESTINATION_CONFLICT = -6, /* buffers that must not overlap do         */
  MOE_ERR_HIP = -7                   /* the HIP runtime reported an error        */
} moe_status;

/* Router score functions. */
enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 };

/* Element types. */
enum {
  MOE_DTYPE_BF16 = 0,  /* bfloat16                                              */
  MOE_DTYPE_F32 = 1,   /* float32                                               */
  MOE_DTYPE_MXFP4 = 2, /* e2m1 pairs (low nibble = even element) + one E8M0 scale
                          byte per 32 elements along the reduction dimension    */
  MOE_DTYPE_FP8_E4M3 = 3, /* OCP FP8 E4M3 (bias 7, largest 448) codes + one fp32
                          scale per row (weights: per output channel)           */
  MOE_DTYPE_FP8_BLOCK = 4 /* E4M3 weight codes + one fp32 scale per 128 x 128 block
                          (block_shape [128, 128])                              */
};

/* Activations of GEMM1 (page "modular_kernel.py", activation(): the output is
 * half as wide as GEMM1's; "silu" gives silu(first half) * second half and
 * "gelu" gelu(first half) * second half).  silu(g) = g / (1 + e^-g);
 * gelu(g) = g/2 * (1 + erf(g / sqrt 2)), the erf form. */
enum { MOE_ACT_SILU = 0, MOE_ACT_GELU = 1 };

/* Options of the fused entry points; NULL (or all fields 0) gives the
 * defaults.
 *   activation        MOE_ACT_SILU or MOE_ACT_GELU, for every expert MLP
 *                     (the shared expert's included)
 *   activation_clamp  0: none.  > 0: before the product the gate is limited
 *                     to <= clamp and the up value to [-clamp, clamp] (the
 *                     activation_clamp of the fused SwiGLU epilogue, page
 *                     "flashinfer_moe_ep.py", build_fi_mega_config).  Must be
 *                     finite and >= 0.
 *   apply_router_weight_on_input  nonzero: the routing weight scales each
 *                     token row before GEMM1 (rounded to bf16) and the combine
 *                     adds the expert rows unweighted (page
 *                     "modular_kernel.py", forward(), prepare() and
 *                     finalize()).  top_k must be 1.  The deferred form then
 *                     returns expert_weights of exactly 1.
 *   chunk_tokens      0: one pass over all T tokens.  > 0: moe_fused_experts
 *                     runs the layer over consecutive chunks of at most this
 *                     many tokens, reusing one workspace sized for a chunk
 *                     (the activation chunking of forward(), page
 *                     "modular_kernel.py").  The deferred form takes no
 *                     chunking: chunk_tokens must be 0 or >= T there.
 *   batched_max_tokens 0: the standard permuted layout.  > 0: the batched
 *                     experts format (page "modular_kernel.py",
 *                     FusedMoEActivationFormat.BatchedExperts) with this many
 *                     rows per local expert, as moe_permute_batched lays out;
 *                     the deferred form's gemm2_permuted then has
 *                     E_l * batched_max_tokens rows (R_pad at least that), and
 *                     routes past an expert's capacity are dropped (map -1).
 *                     A capacity of T never drops a route. */
typedef struct moe_layer_options {
  int32_t activation;
  float activation_clamp;
  int32_t apply_router_weight_on_input;
  int32_t chunk_tokens;
  int32_t batched_max_tokens;
  int32_t act_quant;        /* MOE_QUANT_NONE, MOE_QUANT_FP8 (FP8 or MXFP4 weights),
                               MOE_QUANT_FP8X2 (MXFP4 weights) or MOE_QUANT_FP8_BLOCK
                               (FP8_BLOCK weights) */
  const float* a1_scale;    /* (device) static scale of the GEMM1 input, or NULL */
  const float* a2_scale;    /* (device) static scale of the GEMM2 input, or NULL */
} moe_layer_options;

/* Activation quantization of the fused calls (quant_dtype and
 * per_act_token_quant of page "modular_kernel.py"): MOE_QUANT_FP8 quantizes
 * each token row to FP8 E4M3 before dispatch (moe_quantize_fp8, one scale per
 * row, or the static a1_scale) and each bf16 hidden row before GEMM2 (per row,
 * or a2_scale); both GEMMs then multiply FP8 codes on the matrix cores and
 * apply the row (and FP8 weights' channel) scales in fp32.  Needs FP8 weights
 * (H and I multiples of 128) or MXFP4 weights (multiples of 256: FP8 x e2m1
 * on the matrix cores, the E8M0 block scales applied by them); the shared
 * expert stays bf16.  In the standard layout GEMM1 reads the quantized token
 * rows through the permute's inverse map (no gather); in the batched experts
 * format the quantized rows are gathered into the capacity blocks. */
/* MOE_QUANT_FP8X2 keeps bf16 activations close to bf16 precision on the
 * FP8 x e2m1 matrix cores: each row becomes two E4M3 terms with one scale,
 * x ~ scale * (q1 + q2 / 16) (moe_quantize_fp8x2), before dispatch and before
 * GEMM2, and both GEMMs multiply both terms by the e2m1 weights.  Needs MXFP4
 * weights (H and I multiples of 256) and dynamic scales (a1_scale and a2_scale
 * NULL); either layout. */
/* MOE_QUANT_FP8_BLOCK: blockwise FP8 (block_shape [128, 128] with
 * per_act_token_quant, page "modular_kernel.py", FusedMoEPermuteExpertsUnpermute
 * quant properties): each token row, and each bf16 hidden row before GEMM2,
 * is quantized per group of 128 consecutive elements (moe_quantize_fp8_blockwise),
 * and both GEMMs apply one activation scale per row and 128 k and one weight
 * scale per 128 x 128 block to each k-block's sum.  Needs MOE_DTYPE_FP8_BLOCK
 * weights, H and I multiples of 128, dynamic scales and no router weight on
 * the input; either layout (the quantized rows are always gathered). */
enum { MOE_QUANT_NONE = 0, MOE_QUANT_FP8 = 1, MOE_QUANT_FP8X2 = 2, MOE_QUANT_FP8_BLOCK = 3 };

/* Expert weights of one GEMM, all local experts, reduction dimension last:
 *   BF16:  data = bf16 [E_l, N, K],   scales = NULL
 *   MXFP4: data = u8 [E_l, N, K/2],   scales = u8 [E_l, N, K/32]
 *   FP8:   data = e4m3 [E_l, N, K],   scales = fp32 [E_l, N] (per output
 *          channel, per_out_ch_quant of page "modular_kernel.py"); these
 *          multiply FP8 activations only (the *_fp8 GEMMs, or MOE_QUANT_FP8)
 *   FP8_BLOCK: data = e4m3 [E_l, N, K], scales = fp32 [E_l, N/128, K/128]
 *          (block_shape [128, 128]; element (n, k) is code * scale[n/128][k/128]);
 *          these multiply blockwise FP8 activations only (the *_fp8_blockwise
 *          GEMMs, or MOE_QUANT_FP8_BLOCK); N and K multiples of 128
 * (GEMM1: N = 2I, K = H, rows [0, I) gate and [I, 2I) up; GEMM2: N = H, K = I.)
 * The tag matters: a buffer read as a wider type than it holds is garbage
 * (page "moe_output.py", the comment on expert_weights). */
typedef struct moe_weights {
  int32_t dtype;
  const void* data;      /* (device) */
  const void* scales;    /* (device) MXFP4 and FP8 only */
} moe_weights;

/* Text of a status code (static storage). */
const char* moe_status_string(int status);

/* Message of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

/* Padded permuted row count this library uses for T tokens and top_k k:
 * T*k rounded up to a multiple of 128 (0 for T = 0).  Any R_pad >= T*k is
 * accepted; rows at or past the local route count are never read
 * (page "moe_output.py": the padded row count is never referenced). */
int64_t moe_permuted_rows(int64_t T, int32_t k);

/* Workspace bytes moe_fused_experts (shared expert of intermediate shared_I,
 * 0 for none) and moe_fused_experts_unfinalized (shared_I = 0) need for this
 * problem with these options (NULL: defaults): sized for one chunk when
 * chunking, for E_l * batched_max_tokens rows in the batched experts format.
 * Host-only arithmetic.  Returns MOE_ERR_INVALID_ARGUMENT on bad sizes.
 * Mirrors FusedMoEPermuteExpertsUnpermute.workspace_shapes (page
 * "modular_kernel.py"): the caller allocates, the library reuses. */
int moe_workspace_size(int64_t T, int32_t k, int32_t E, int32_t E_l, int32_t H, int32_t I,
                       int32_t w_dtype, int32_t shared_I, const moe_layer_options* options,
                       size_t* bytes);

/* Router ([Router] stage).  For each token t the k experts with the largest
 * logits, ordered by logit descending, ties to the smaller expert id, and
 * their weights:
 *   SOFTMAX: p = softmax over all E logits;   SIGMOID: p_e = 1/(1+exp(-l_e));
 *   renormalize != 0: w_j = p_j / sum over the k selected p;  else w_j = p_j;
 *   then w_j *= rsf (the routed scaling factor, folded into the weights as the
 *   expert_weights comment of page "moe_output.py" describes).
 *   logits       (device) fp32 [T, E]
 *   topk_ids     (device) int32 [T, k]  out
 *   topk_weights (device) fp32 [T, k]   out
 * Limits: 1 <= k <= min(E, 32), E <= 1024. */
int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t score_fn,
                   int32_t renormalize, float rsf, int32_t* topk_ids, float* topk_weights,
                   void* stream);

/* Permute (single-GPU part of [Quantize-Dispatch]; prepare() of page
 * "modular_kernel.py" with its expert_map and per-local-expert counts).
 *   L(t,j) = expert_map[topk_ids[t,j]] (or topk_ids[t,j] when expert_map is
 *   NULL); L = -1 marks an expert that is not local.
 *   offsets[e] = number of local routes to local experts < e, e in [0, E_l];
 *   offsets[E_l] = R_l.
 *   map[t,j] = offsets[L] + (number of routes (t',j') to L with t'*k+j' <
 *   t*k+j), or -1 when L = -1 (page "moe_output.py",
 *   expanded_idx_to_permuted_idx).  The order is stable and deterministic.
 *   inv[r] = t*k+j of the route placed in row r, for r < R_l; -1 for
 *   R_l <= r < R_pad.
 *   x_perm[r, :] = x[inv[r] / k, :] for r < R_l; rows >= R_l are not written.
 *   With x_weights (apply_router_weight_on_input of prepare(), page
 *   "modular_kernel.py": the routing weights go on the activations before
 *   dispatch), x_perm[map[t,j], :] = bf16(x_weights[t,j] * x[t, :]).
 *   topk_ids   (device) int32 [T, k]; an id outside [0, E) is a caller error
 *              and is treated as a non-local route
 *   expert_map (device) int32 [E] with entries in [-1, E_l), or NULL (E_l = E)
 *   x          (device) bf16 [T, H]
 *   map        (device) int32 [T, k]      out
 *   offsets    (device) int32 [E_l + 1]   out
 *   inv        (device) int32 [R_pad]     out, may be NULL
 *   x_perm     (device) bf16 [R_pad, H]   out, may be NULL (no gather)
 *   x_weights  (device) fp32 [T, k] or NULL (rows copied unscaled)
 *   workspace  (device) scratch of moe_workspace_size() bytes, may be NULL
 *              when workspace_bytes is 0 (this version needs none)
 * Limits: E_l <= 1024, H a multiple of 8. */
int moe_permute(const int32_t* topk_ids, const int32_t* expert_map, int64_t T, int32_t k,
                int32_t E, int32_t E_l, const void* x, int32_t H, int64_t R_pad, int32_t* map,
                int32_t* offsets, int32_t* inv, void* x_perm, const float* x_weights,
                void* workspace, size_t workspace_bytes, void* stream);

/* Router and Permute map in one call ([Router] followed by the permute of
 * [Quantize-Dispatch], prepare() of page "modular_kernel.py"): the topk ids
 * and weights of moe_route_topk, then the map, offsets and inverse map of
 * moe_permute with x_perm = NULL (no rows are gathered: the gathered form of
 * GEMM1 reads them through inv).  The results are those of the two calls.
 * For T <= 16 both steps run in one kernel of one workgroup (each wave
 * routes one token and keeps its local experts in on-chip memory, then the
 * workgroup sorts them), which saves a launch on decode batches; larger
 * batches launch the two kernels.
 *   logits, topk_ids, topk_weights   as for moe_route_topk
 *   expert_map, map, offsets, inv    as for moe_permute
 * Limits: those of both calls. */
int moe_route_permute(const float* logits, int64_t T, int32_t E, int32_t k, int32_t score_fn,
                      int32_t renormalize, float rsf, const int32_t* expert_map, int32_t E_l,
                      int64_t R_pad, int32_t* topk_ids, float* topk_weights, int32_t* map,
                      int32_t* offsets, int32_t* inv, void* stream);

/* Router, permute map and GEMM1 in one call ([Router], the permute of
 * [Quantize-Dispatch] and the first expert GEMM with its activation; page
 * "modular_kernel.py", prepare() and apply()): moe_route_permute followed by
 * moe_grouped_gemm1_act_gathered(x, inv, T, k, offsets, ..., h).  The results
 * are those of the two calls.  With bf16 weights, at most 8 tokens and 64
 * routes, and few rows per local expert (R_pad / E_l under 16), the three
 * steps run in one kernel: every workgroup routes the tokens and sorts the
 * routes in on-chip memory itself, then runs its share of GEMM1 on the token
 * rows through that inverse map (one launch instead of two on decode
 * batches); otherwise the router-permute and GEMM1 kernels are launched.
 *   logits, topk_ids, topk_weights          as for moe_route_topk
 *   expert_map, R_pad, map, offsets, inv    as for moe_permute (inv required)
 *   x, H, I, w1, activation, activation_clamp, h, workspace
 *                                           as for moe_grouped_gemm1_act_gathered
 * Limits: those of the calls it stands for. */
int moe_route_permute_gemm1_act(const float* logits, const void* x, int64_t T, int32_t H,
                                int32_t I, int32_t E, int32_t E_l, int32_t k, int32_t score_fn,
                                int32_t renormalize, float rsf, const int32_t* expert_map,
                                int64_t R_pad, const moe_weights* w1, int32_t activation,
                                float activation_clamp, int32_t* topk_ids, float* topk_weights,
                                int32_t* map, int32_t* offsets, int32_t* inv, void* h,
                                void* workspace, size_t workspace_bytes, void* stream);

/* FP8 E4M3 quantization of bf16 rows (the quantize half of [Quantize-Dispatch];
 * prepare() of page "modular_kernel.py" with per_act_token_quant, or a static
 * a1_scale / a2_scale).  Per row, in fp32:
 *   dynamic (static_scale NULL): a = max |x| (448 for an all-zero row),
 *     inv = 448 / a, scale = a / 448;   static: scale = *static_scale, inv = 1 / scale;
 *   q[j] = E4M3 code nearest to clamp(x[j] * inv, -448, 448), ties to even.
 * With row_weights (fp32 [rows], apply_router_weight_on_input) the row is
 * first bf16(row_weights[r] * x).
 *   x         (device) bf16 [rows, H];   q (device) u8 [rows, H] out
 *   row_count (device) int32 scalar or NULL: only rows < *row_count are
 *             quantized (the local routes of permuted rows: offsets + E_l)
 *   scales  (device) fp32 [rows] out (the static scale repeated when given)
 * Limits: H a multiple of 16. */
int moe_quantize_fp8(const void* x, int64_t rows, int32_t H, const float* static_scale,
                     const float* row_weights, const int32_t* row_count, uint8_t* q,
                     float* scales, void* stream);

/* Permute with FP8 rows (the dispatch half of [Quantize-Dispatch]): as
 * moe_permute, gathering the quantized rows and their scales:
 *   xq_perm[map[t,j], :] = xq[t, :],  xq_perm_scales[map[t,j]] = x_scales[t].
 *   xq (device) u8 [T, H], x_scales (device) fp32 [T] (from moe_quantize_fp8)
 *   xq_perm (device) u8 [R_pad, H] out, xq_perm_scales (device) fp32 [R_pad] out
 * Limits: H a multiple of 16. */
int moe_permute_fp8(const int32_t* topk_ids, const int32_t* expert_map, int64_t T, int32_t k,
                    int32_t E, int32_t E_l, const uint8_t* xq, const float* x_scales, int32_t H,
                    int64_t R_pad, int32_t* map, int32_t* offsets, int32_t* inv, uint8_t* xq_perm,
                    float* xq_perm_scales, void* stream);

/* The two grouped GEMMs on FP8 rows with FP8 weights (apply() of page
 * "modular_kernel.py" with a1q_scale / a2_scale and w1_scale / w2_scale):
 *   C[r, n] = a_scale[r] * w_scale[e, n] * sum_k a[r, k] * W[e, n, k]
 * (E4M3 products summed exactly in fp32 by the 32x32x64 MFMA), then, for
 * GEMM1, act(gate) * up and one rounding to bf16.
 *   a_perm / h_perm  (device) u8 [R_pad, H or I];  a_scales / h_scales fp32 [R_pad]
 *   w1 / w2          MOE_DTYPE_FP8_E4M3 weights, or MOE_DTYPE_MXFP4 (then
 *                    C[r, n] = a_scale[r] * sum_k a[r, k] * e2m1[n, k] * 2^(e8m0 - 127),
 *                    the block scales applied by the matrix cores)
 *   h / y            (device) bf16 [R_pad, I or H] out
 *   workspace        as for the bf16 calls
 * Limits: H and I multiples of 128 (FP8 weights) or 256 (MXFP4 weights). */
int moe_grouped_gemm1_act_fp8(const uint8_t* a_perm, const float* a_scales,
                              const int32_t* offsets, int32_t E_l, int64_t R_pad, int32_t H,
                              int32_t I, const moe_weights* w1, int32_t activation,
                              float activation_clamp, void* h, void* workspace,
                              size_t workspace_bytes, void* stream);
int moe_grouped_gemm2_fp8(const uint8_t* h_perm, const float* h_scales, const int32_t* offsets,
                          int32_t E_l, int64_t R_pad, int32_t I, int32_t H, const moe_weights* w2,
                          void* y, void* workspace, size_t workspace_bytes, void* stream);

/* Blockwise FP8 E4M3 quantization of bf16 rows (the quantize half of
 * [Quantize-Dispatch] with block_shape [128, 128] and per_act_token_quant,
 * page "modular_kernel.py"): every group of 128 consecutive elements of a row
 * gets its own scale by the rule of moe_quantize_fp8 (dynamic: a = max |x|
 * over the group, 448 for an all-zero group; inv = 448 / a; scale = a / 448;
 * q = E4M3 nearest to clamp(x * inv, -448, 448), ties to even).
 *   x          (device) bf16 [rows, H]
 *   row_count  (device) int32 scalar or NULL: only rows < *row_count
 *   q          (device) u8 [rows, H] out
 *   scales     (device) fp32 [H / 128, scales_ld] out, group-major: the scale
 *              of row r, group g at scales[g * scales_ld + r]; scales_ld >= rows
 * Limits: H a multiple of 128. */
int moe_quantize_fp8_blockwise(const void* x, int64_t rows, int32_t H, const int32_t* row_count,
                               uint8_t* q, float* scales, int64_t scales_ld, void* stream);

/* moe_permute on blockwise FP8 rows: as moe_permute_fp8, the group scales
 * gathered along with the codes:
 *   xq_perm[map[t,j], :] = xq[t, :],
 *   xq_perm_scales[g * R_pad + map[t,j]] = x_scales[g * T + t]   (g < H / 128)
 *   xq        (device) u8 [T, H];  x_scales (device) fp32 [H / 128, T]
 *   xq_perm   (device) u8 [R_pad, H] out;  xq_perm_scales (device) fp32 [H / 128, R_pad] out
 * Limits: H a multiple of 128. */
int moe_permute_fp8_blockwise(const int32_t* topk_ids, const int32_t* expert_map, int64_t T,
                              int32_t k, int32_t E, int32_t E_l, const uint8_t* xq,
                              const float* x_scales, int32_t H, int64_t R_pad, int32_t* map,
                              int32_t* offsets, int32_t* inv, uint8_t* xq_perm,
                              float* xq_perm_scales, void* stream);

/* The two grouped GEMMs on blockwise FP8 rows with MOE_DTYPE_FP8_BLOCK weights
 * (apply() of page "modular_kernel.py" with block_shape [128, 128]):
 *   C[r, n] = sum over k-blocks b of a_scale[b][r] * w_scale[e][n/128][b] *
 *             sum_{k in block b} a[r, k] * W[e, n, k]
 * (each block's E4M3 products summed in fp32 by the 32x32x64 MFMA, scaled and
 * added in fp32), then, for GEMM1, act(gate) * up and one rounding to bf16.
 *   a_perm / h_perm    (device) u8 [R_pad, H or I]
 *   a_scales / h_scales (device) fp32 [H/128 or I/128, R_pad], group-major
 *                      (as moe_permute_fp8_blockwise / moe_quantize_fp8_blockwise
 *                      with scales_ld = R_pad write them)
 *   h / y              (device) bf16 [R_pad, I or H] out;  workspace as for
 *                      the bf16 calls
 * Limits: H and I multiples of 128. */
int moe_grouped_gemm1_act_fp8_blockwise(const uint8_t* a_perm, const float* a_scales,
                                        const int32_t* offsets, int32_t E_l, int64_t R_pad,
                                        int32_t H, int32_t I, const moe_weights* w1,
                                        int32_t activation, float activation_clamp, void* h,
                                        void* workspace, size_t workspace_bytes, void* stream);
int moe_grouped_gemm2_fp8_blockwise(const uint8_t* h_perm, const float* h_scales,
                                    const int32_t* offsets, int32_t E_l, int64_t R_pad,
                                    int32_t I, int32_t H, const moe_weights* w2, void* y,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* FP8 GEMM1 + activation reading its rows straight from the quantized token
 * rows (the dispatch of [Quantize-Dispatch] folded into the first expert GEMM;
 * apply() of page "modular_kernel.py"): the same result as moe_permute_fp8 (or
 * the two-term rows dispatched by it) followed by moe_grouped_gemm1_act_fp8 or
 * moe_grouped_gemm1_act_fp8x2, bit for bit, without the gather.  Permuted row
 * r of expert e reads token row inv[r] / k and that token's scale.
 *   xq        (device) u8 [T, H * terms]: FP8 codes (terms 1) or two-term codes
 *             (terms 2, moe_quantize_fp8x2) of the tokens
 *   x_scales  (device) fp32 [T], one per token
 *   inv       (device) int32 [R_pad] from moe_permute (rows < offsets[E_l] read)
 *   offsets, E_l, R_pad, H, I, activation, h, workspace: as for
 *             moe_grouped_gemm1_act_fp8; w1 FP8 or MXFP4 weights (terms 1),
 *             MXFP4 (terms 2)
 * Limits: as for moe_grouped_gemm1_act_fp8; xq at most 4 GiB. */
int moe_grouped_gemm1_act_fp8_gathered(const uint8_t* xq, const float* x_scales,
                                       int32_t terms, const int32_t* inv, int64_t T, int32_t k,
                                       const int32_t* offsets, int32_t E_l, int64_t R_pad,
                                       int32_t H, int32_t I, const moe_weights* w1,
                                       int32_t activation, float activation_clamp, void* h,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Two-term FP8 E4M3 quantization of bf16 rows, for bf16 activations on the
 * FP8 x e2m1 matrix cores with MXFP4 weights (the quantize half of
 * [Quantize-Dispatch], page "modular_kernel.py", prepare(), per token).  Per
 * row, in fp32: a = max |x| (448 for an all-zero row), inv = 448 / a,
 * scale = a / 448; for each element v = clamp(x[j] * inv, -448, 448),
 *   q1 = E4M3 code nearest to v (ties to even),
 *   q2 = E4M3 code nearest to 16 * (v - value(q1))   (the residual is exact),
 * so x[j] ~ scale * (value(q1) + value(q2) / 16).  With row_weights the row is
 * first bf16(row_weights[r] * x).
 *   x         (device) bf16 [rows, H]
 *   q         (device) u8 [rows, 2H] out: per 64 k, the 64 codes q1 of those
 *             k, then their 64 codes q2
 *   row_count (device) int32 scalar or NULL, as for moe_quantize_fp8
 *   scales    (device) fp32 [rows] out
 * The rows are dispatched with moe_permute_fp8 as rows of 2H bytes.
 * Limits: H a multiple of 64. */
int moe_quantize_fp8x2(const void* x, int64_t rows, int32_t H, const float* row_weights,
                       const int32_t* row_count, uint8_t* q, float* scales, void* stream);

/* The two grouped GEMMs on two-term FP8 rows (moe_quantize_fp8x2) with MXFP4
 * weights (apply() of page "modular_kernel.py"):
 *   C[r, n] = a_scale[r] * sum_k (q1[r, k] + q2[r, k] / 16) * e2m1[n, k] * 2^(e8m0 - 127)
 * (two scaled 32x32x64 MFMAs per 64 k, the second with A scale 2^-4), then,
 * for GEMM1, act(gate) * up and one rounding to bf16.
 *   a_perm / h_perm  (device) u8 [R_pad, 2H or 2I];  a_scales / h_scales fp32 [R_pad]
 *   w1 / w2          MOE_DTYPE_MXFP4 weights
 *   h / y            (device) bf16 [R_pad, I or H] out;  workspace as for the bf16 calls
 * Limits: H and I multiples of 256. */
int moe_grouped_gemm1_act_fp8x2(const uint8_t* a_perm, const float* a_scales,
                                const int32_t* offsets, int32_t E_l, int64_t R_pad, int32_t H,
                                int32_t I, const moe_weights* w1, int32_t activation,
                                float activation_clamp, void* h, void* workspace,
                                size_t workspace_bytes, void* stream);
int moe_grouped_gemm2_fp8x2(const uint8_t* h_perm, const float* h_scales,
                            const int32_t* offsets, int32_t E_l, int64_t R_pad, int32_t I,
                            int32_t H, const moe_weights* w2, void* y, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Permute into the batched experts format (page "modular_kernel.py":
 * FusedMoEActivationFormat.BatchedExperts, activations laid out as (local
 * experts, max tokens per expert, hidden), with the per-local-expert token
 * counts that prepare() returns as expert_num_tokens).
 *   Expert L owns rows [L * max_tokens, (L + 1) * max_tokens).  Walking the
 *   expanded index t*k+j upward, the n-th route to L takes row
 *   L * max_tokens + n while n < max_tokens; a route past that capacity, or
 *   to an expert that is not local, gets map -1.
 *   expert_num_tokens[L] = all routes to L (above max_tokens exactly when
 *   routes were dropped); the GEMMs use min(expert_num_tokens[L], max_tokens).
 *   x_batched[map[t,j], :] = x[t, :] (or bf16(x_weights[t,j] * x[t, :])); rows
 *   past an expert's count are not written.
 *   topk_ids, expert_map, x, x_weights: as for moe_permute
 *   map               (device) int32 [T, k] out
 *   expert_num_tokens (device) int32 [E_l] out (written even for T = 0)
 *   x_batched         (device) bf16 [E_l, max_tokens, H] out, or NULL
 * Limits: E_l * max_tokens < 2^31, H a multiple of 8. */
int moe_permute_batched(const int32_t* topk_ids, const int32_t* expert_map, int64_t T, int32_t k,
                        int32_t E, int32_t E_l, const void* x, int32_t H, int32_t max_tokens,
                        int32_t* map, int32_t* expert_num_tokens, void* x_batched,
                        const float* x_weights, void* stream);

/* Grouped GEMM1 + activation (apply() and activation() of page
 * "modular_kernel.py").  For every local expert e and row r in
 * [offsets[e], offsets[e+1]):
 *   g = a_perm[r, :] . W1[e, n, :],  u = a_perm[r, :] . W1[e, I + n, :]
 *   h[r, n] = act(g) * u   (fp32 accumulation, one rounding to bf16)
 *   activation        MOE_ACT_SILU or MOE_ACT_GELU
 *   activation_clamp  0, or > 0 to clamp g and u first (moe_layer_options)
 *   a_perm  (device) bf16 [R_pad, H]
 *   offsets (device) int32 [E_l + 1] as written by moe_permute
 *   w1      GEMM1 weights, N = 2I, K = H (BF16, or MXFP4: the decoded values
 *           are exact in bf16, so the MFMAs run in bf16 either way)
 *   h       (device) bf16 [R_pad, I] out; rows >= offsets[E_l] not written
 *   workspace (device) optional scratch, 256-byte aligned, not overlapping
 *           a_perm or h; NULL with workspace_bytes 0 is valid.  With
 *           moe_grouped_gemm_workspace_size(R_pad, I, 1) bytes, calls whose
 *           experts have few rows split the reduction over H into pieces
 *           summed in a fixed order (results are the same on every run);
 *           with less, fewer pieces or none.  Calls with many rows use it
 *           when their tiles leave a last round of a few tiles: those tiles
 *           are split the same way, so that round fills the GPU.
 * Limits: H and I multiples of 64; R_pad >= offsets[E_l].  MXFP4 weights
 * without scales, or bf16 weights with scales, are MOE_ERR_INVALID_ARGUMENT. */
int moe_grouped_gemm1_act(const void* a_perm, const int32_t* offsets, int32_t E_l, int64_t R_pad,
                          int32_t H, int32_t I, const moe_weights* w1, int32_t activation,
                          float activation_clamp, void* h, void* workspace,
                          size_t workspace_bytes, void* stream);

/* GEMM1 + activation reading its rows straight from the token matrix (the
 * dispatch of [Quantize-Dispatch] folded into the first expert GEMM; apply()
 * of page "modular_kernel.py"): the same result as moe_permute's gather
 * followed by moe_grouped_gemm1_act, bit for bit, without the x_perm round
 * trip.  Permuted row r of expert e reads x[inv[r] / k, :].
 *   x        (device) bf16 [T, H] token rows (T * H * 2 bytes at most 4 GiB)
 *   inv      (device) int32 [R_pad] from moe_permute (row -> expanded index
 *            t*k + j for r < offsets[E_l]; other rows are never read)
 *   offsets, E_l, R_pad, H, I, w1, activation, h, workspace: as for
 *            moe_grouped_gemm1_act (bf16 or MXFP4 weights).
 * The fused calls use it for every pass of bf16 activations in the standard
 * layout with the weights not on the input (x at most 4 GiB): it saves the
 * gather kernel and the x_perm write and re-read. */
int moe_grouped_gemm1_act_gathered(const void* x, const int32_t* inv, int64_t T, int32_t k,
                                   const int32_t* offsets, int32_t E_l, int64_t R_pad, int32_t H,
                                   int32_t I, const moe_weights* w1, int32_t activation,
                                   float activation_clamp, void* h, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Grouped GEMM2 (apply() of page "modular_kernel.py"; its output is the
 * unweighted, unreduced gemm2_permuted of page "moe_output.py": densely
 * packed at H).  For every local expert e and row r in [offsets[e],
 * offsets[e+1]):  y[r, n] = h[r, :] . W2[e, n, :]  (fp32 accumulation, bf16).
 *   h       (device) bf16 [R_pad, I]
 *   w2      GEMM2 weights, N = H, K = I
 *   y       (device) bf16 [R_pad, H] out; rows >= offsets[E_l] not written
 *   workspace as for moe_grouped_gemm1_act, with
 *           moe_grouped_gemm_workspace_size(R_pad, H, 0) bytes
 * Limits: H and I multiples of 64. */
int moe_grouped_gemm2(const void* h, const int32_t* offsets, int32_t E_l, int64_t R_pad,
                      int32_t I, int32_t H, const moe_weights* w2, void* y, void* workspace,
                      size_t workspace_bytes, void* stream);

/* The two grouped GEMMs in the batched experts format (apply() of page
 * "modular_kernel.py" with its expert_num_tokens): the same arithmetic as
 * moe_grouped_gemm1_act / moe_grouped_gemm2 on expert e's rows
 * [e * max_tokens, e * max_tokens + min(expert_num_tokens[e], max_tokens)).
 *   a_batched / h_batched / y_batched  (device) bf16 [E_l, max_tokens, H or I]
 *   expert_num_tokens  (device) int32 [E_l]
 *   max_rows   an upper bound on the rows to compute that the caller knows
 *              (T * top_k), or 0 for E_l * max_tokens; it only picks the tile
 *              shape
 *   workspace  as for the standard calls, with
 *              moe_grouped_gemm_workspace_size(E_l * max_tokens, ...) bytes
 * Rows past an expert's count are neither read nor written. */
int moe_grouped_gemm1_act_batched(const void* a_batched, const int32_t* expert_num_tokens,
                                  int32_t E_l, int32_t max_tokens, int64_t max_rows, int32_t H,
                                  int32_t I, const moe_weights* w1, int32_t activation,
                                  float activation_clamp, void* h_batched, void* workspace,
                                  size_t workspace_bytes, void* stream);
int moe_grouped_gemm2_batched(const void* h_batched, const int32_t* expert_num_tokens,
                              int32_t E_l, int32_t max_tokens, int64_t max_rows, int32_t I,
                              int32_t H, const moe_weights* w2, void* y_batched, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Fused tail on one GPU: finalize, the shared-expert add, the residual add
 * and the next layer's RMSNorm in one pass (page "moe_output.py", MoEOutput
 * docstring: the code after the layer, usually the next layer's
 * normalization, may finish the layer's open reduction).
 * For every token t, with z the fp32 sum
 *   z[t, :] = rsf_fin * sum_{j: map>=0} w[t,j] * y_perm[map[t,j], :]
 *             + shared[t, :] + residual[t, :]
 *   residual[t, :] = bf16(z[t, :])                                  (in place)
 *   out[t, :] = bf16(z[t, :] / sqrt(mean(z[t, :]^2) + eps) * gamma[:])
 * (the norm uses z before the residual's rounding).
 *   y_perm, y_rows, weights, weights_dtype, map, T, k, H, rsf_fin, shared:
 *              as for moe_finalize (weights may be NULL)
 *   residual   (device) bf16 [T, H] in/out (the residual stream)
 *   gamma      (device) bf16 [H] the norm's per-column scale
 *   eps        >= 0
 *   out        (device) bf16 [T, H] out; must not overlap residual, shared
 *              or y_perm; shared must not overlap residual
 * Limits: H a multiple of 8, at most 16384. */
int moe_finalize_add_rmsnorm(const void* y_perm, int64_t y_rows, const void* weights,
                             int32_t weights_dtype,
                             const int32_t* map, int64_t T, int32_t k, int32_t H, float rsf_fin,
                             const void* shared, void* residual, const void* gamma, float eps,
                             void* out, void* stream);

/* Scratch bytes with which a grouped GEMM of R_pad permuted rows and N_out
 * output columns (gated != 0: GEMM1, whose weights have 2 N_out rows) may
 * split its reduction as far as it ever does: fp32 slices of all rows for
 * few-row calls (up to 16 within 64 MiB), or fp32 tiles for the pieces of a
 * short last round (32 MiB and 1 KiB), whichever is larger.  Host-only
 * arithmetic.  MOE_ERR_INVALID_ARGUMENT on bad sizes. */
int moe_grouped_gemm_workspace_size(int64_t R_pad, int32_t N_out, int32_t gated, size_t* bytes);

/* Finalize (finalize() of page "modular_kernel.py"; MoEOutput of page
 * "moe_output.py": the routed scaling factor multiplies the routed sum before
 * the shared-expert add).
 *   out[t, :] = rsf_fin * sum_{j ascending, map[t,j] >= 0} w[t,j] * y[map[t,j], :]
 *               + shared[t, :]
 * fp32 accumulation, one rounding to bf16.  -1 entries, and entries at or
 * past y_rows, are skipped, so no row outside y_perm is read.  Every row of
 * out is written (a token with no local route gets 0, or its shared row).
 *   y_perm   (device) bf16 [y_rows, H]: R_pad rows in the standard layout,
 *            E_l * max_tokens in the batched experts format; may be NULL when
 *            y_rows is 0
 *   y_rows   its row count (>= 0)
 *   weights  (device) [T, k] of weights_dtype (MOE_DTYPE_F32 or MOE_DTYPE_BF16),
 *            or NULL: every weight is 1 (finalize() with
 *            apply_router_weight_on_input, whose weights went on the inputs)
 *   map      (device) int32 [T, k]
 *   shared   (device) bf16 [T, H] or NULL
 *   out      (device) bf16 [T, H] out; may alias shared exactly (in place),
 *            must not overlap y_perm's y_rows rows
 * Limits: H a multiple of 8, k <= 32. */
int moe_finalize(const void* y_perm, int64_t y_rows, const void* weights, int32_t weights_dtype,
                 const int32_t* map, int64_t T, int32_t k, int32_t H, float rsf_fin,
                 const void* shared, void* out, void* stream);

/* Deferred-finalize form (UnfinalizedMoEOutput of page "moe_output.py"): the
 * router, permute and both GEMMs, stopping before the top-k reduction.
 *   logits          (device) fp32 [T, E];  x (device) bf16 [T, H]
 *   expert_map      (device) int32 [E] or NULL
 *   gemm2_permuted  (device) bf16 [R_pad, H] out (unweighted GEMM2 rows)
 *   expert_weights  (device) bf16 [T, k] out (the activation dtype, since this
 *                   call routes itself), rsf already applied
 *   map             (device) int32 [T, k] out (-1 = expert not local)
 *   workspace       (device) >= moe_workspace_size(..., 0, options) bytes,
 *                   256-byte aligned
 * A deferred call takes no destination for the finalized output; pass the
 * three buffers to moe_finalize (weights_dtype MOE_DTYPE_BF16) later. */
int moe_fused_experts_unfinalized(const float* logits, const void* x, int64_t T, int32_t H,
                                  int32_t I, int32_t E, int32_t E_l, int32_t k, int32_t score_fn,
                                  int32_t renormalize, float rsf, const int32_t* expert_map,
                                  const moe_weights* w1, const moe_weights* w2,
                                  const moe_layer_options* options, int64_t R_pad,
                                  void* gemm2_permuted, void* expert_weights, int32_t* map,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device memory moe_fused_experts_unfinalized_noalloc uses as its
 * scratch: a static array the library holds on every device it runs on,
 * from the library's first use there until the process ends. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)

/* The deferred form without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Arguments, results and errors are those of
 * moe_fused_experts_unfinalized (less the workspace), except:
 *   - the scratch is the library's static array of MOE_NOALLOC_SCRATCH_BYTES
 *     on the current device; the call allocates and frees nothing;
 *   - a problem whose scratch, not counting the GEMMs' split-reduction
 *     partials, exceeds that size fails with MOE_ERR_SIZE_MISMATCH (for the
 *     DeepSeek-V3 rank shape, H 7168, I 2048, top_k 8, that is about 3000
 *     tokens); the partials get what is left, so a call may split its GEMMs
 *     into fewer pieces than the workspace form and differ from it in the
 *     last bits (it gives the same bits on every run);
 *   - all calls on one device share the one array: calls that may run at the
 *     same time on one device (other streams, other threads) race.  Each
 *     call writes every scratch byte it reads; none must start at zero. */
int moe_fused_experts_unfinalized_noalloc(const float* logits, const void* x, int64_t T,
                                          int32_t H, int32_t I, int32_t E, int32_t E_l, int32_t k,
                                          int32_t score_fn, int32_t renormalize, float rsf,
                                          const int32_t* expert_map, const moe_weights* w1,
                                          const moe_weights* w2, const moe_layer_options* options,
                                          int64_t R_pad, void* gemm2_permuted,
                                          void* expert_weights, int32_t* map, void* stream);

/* The whole layer, finalized:
 *   out = rsf_fin * sum_j w_j * MLP_{L_j}(x) + shared MLP(x)
 * (with apply_router_weight_on_input: rsf_fin * sum_j MLP_{L_j}(w_j x) + ...)
 * with the shared expert (one dense gated MLP, intermediate shared_I, weights
 * ws1 bf16 [2*shared_I, H] and ws2 bf16 [H, shared_I]) present when
 * shared_I > 0.
 *   options   moe_layer_options or NULL (SiLU, no clamp, one pass)
 *   out       (device) bf16 [T, H]; either x itself (in place, forward()'s
 *             inplace of page "modular_kernel.py") or not overlapping x
 *   workspace (device) >= moe_workspace_size(..., shared_I, options) bytes */
int moe_fused_experts(const float* logits, const void* x, int64_t T, int32_t H, int32_t I,
                      int32_t E, int32_t E_l, int32_t k, int32_t score_fn, int32_t renormalize,
                      float rsf, const int32_t* expert_map, const moe_weights* w1,
                      const moe_weights* w2, int32_t shared_I, const void* ws1, const void* ws2,
                      float rsf_fin, const moe_layer_options* options, void* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Extra workspace bytes moe_fused_experts needs for a shared expert of
 * intermediate size shared_I (0 when shared_I = 0). */
int moe_shared_workspace_size(int64_t T, int32_t H, int32_t shared_I, size_t* bytes);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_MOE_H_ */
