// C ABI of the fused MoE layer: argument checks, workspace layout and the
// call sequences of the fused entry points.  Every check runs on the host
// before anything is enqueued; a failing call enqueues nothing.  The checks
// follow convert_flashinfer_moe_output of vLLM's MoE output contract
// (num_tokens >= 0, top_k > 0, int32 map, T * k elements, one device,
// contiguous buffers, no destination for a deferred output).
#include <algorithm>
#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/moe.h"
#include "moe_common.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool validate_pointers() {
  static int mode = -1;
  if (mode < 0) {
    const char* v = getenv("MOE_VALIDATE");
    mode = (v && v[0] && v[0] != '0') ? 1 : 0;
  }
  return mode == 1;
}

// Under MOE_VALIDATE=1: the pointer must be device memory (or managed).
int check_device_ptr(const void* p, const char* name) {
  if (!p || !validate_pointers()) return MOE_OK;
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(MOE_ERR_DEVICE, "%s is not a HIP allocation", name);
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return fail(MOE_ERR_DEVICE, "%s is not device memory", name);
  return MOE_OK;
}

#define MOE_CHECK(expr)            \
  do {                             \
    int _s = (expr);               \
    if (_s != MOE_OK) return _s;   \
  } while (0)

int need_ptr(const void* p, const char* name) {
  if (!p) return fail(MOE_ERR_INVALID_ARGUMENT, "%s must not be NULL", name);
  if (!aligned16(p)) return fail(MOE_ERR_MISALIGNED, "%s must be 16-byte aligned", name);
  return check_device_ptr(p, name);
}

int opt_ptr(const void* p, const char* name) {
  if (!p) return MOE_OK;
  if (!aligned16(p)) return fail(MOE_ERR_MISALIGNED, "%s must be 16-byte aligned", name);
  return check_device_ptr(p, name);
}

// an optional 4-byte aligned device scalar or array
int opt_ptr4(const void* p, const char* name) {
  if (!p) return MOE_OK;
  if (reinterpret_cast<uintptr_t>(p) & 3u) return fail(MOE_ERR_MISALIGNED, "%s must be 4-byte aligned", name);
  return check_device_ptr(p, name);
}

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return a && b && an && bn && x < y + bn && y < x + an;
}

int check_route_sizes(int64_t T, int32_t E, int32_t k) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "num_tokens must be non-negative (T=%lld)", (long long)T);
  if (k <= 0) return fail(MOE_ERR_INVALID_ARGUMENT, "top_k must be positive (k=%d)", k);
  if (E <= 0 || E > 1024) return fail(MOE_ERR_INVALID_ARGUMENT, "E must be in [1, 1024] (E=%d)", E);
  if (k > E || k > 32) return fail(MOE_ERR_INVALID_ARGUMENT, "top_k must be <= min(E, 32) (k=%d, E=%d)", k, E);
  if (T > (int64_t(1) << 31) / k) return fail(MOE_ERR_INVALID_ARGUMENT, "T * k must fit in int32");
  return MOE_OK;
}

int check_local(int32_t E, int32_t E_l) {
  if (E_l <= 0 || E_l > E || E_l > 1024)
    return fail(MOE_ERR_INVALID_ARGUMENT, "E_l must be in [1, min(E, 1024)] (E_l=%d, E=%d)", E_l, E);
  return MOE_OK;
}

int check_gemm_dims(int32_t H, int32_t I) {
  if (H <= 0 || H % 64) return fail(MOE_ERR_INVALID_ARGUMENT, "H must be a positive multiple of 64 (H=%d)", H);
  if (I <= 0 || I % 64) return fail(MOE_ERR_INVALID_ARGUMENT, "I must be a positive multiple of 64 (I=%d)", I);
  return MOE_OK;
}

int check_weights(const moe_weights* w, const char* name) {
  if (!w) return fail(MOE_ERR_INVALID_ARGUMENT, "%s must not be NULL", name);
  if (w->dtype == MOE_DTYPE_MXFP4 || w->dtype == MOE_DTYPE_FP8_E4M3 ||
      w->dtype == MOE_DTYPE_FP8_BLOCK) {
    MOE_CHECK(need_ptr(w->data, name));
    if (!w->scales) return fail(MOE_ERR_INVALID_ARGUMENT, "%s: %s weights need their scales", name,
                                w->dtype == MOE_DTYPE_MXFP4 ? "MXFP4" : "FP8");
    if (w->dtype != MOE_DTYPE_MXFP4 && (reinterpret_cast<uintptr_t>(w->scales) & 3u))
      return fail(MOE_ERR_MISALIGNED, "%s: FP8 scales must be 4-byte aligned", name);
    return check_device_ptr(w->scales, name);
  }
  if (w->dtype != MOE_DTYPE_BF16) return fail(MOE_ERR_UNSUPPORTED, "%s: unknown weight dtype %d", name, w->dtype);
  if (w->scales) return fail(MOE_ERR_INVALID_ARGUMENT, "%s: bf16 weights take no scales", name);
  return need_ptr(w->data, name);
}

// The weights' scales as the GEMM takes them (NULL for bf16).
const void* scales_of(const moe_weights* w) {
  return w->dtype == MOE_DTYPE_BF16 ? nullptr : w->scales;
}

// FP8 weights multiply FP8 activations only; FP8 activations multiply FP8 or
// MXFP4 weights; block-scaled FP8 weights and blockwise activations pair
// with each other only.
int check_pairing(const moe_weights* w, bool fp8_act, const char* name, bool block = false) {
  if (block != (w->dtype == MOE_DTYPE_FP8_BLOCK))
    return fail(MOE_ERR_INVALID_ARGUMENT,
                "%s: block-scaled FP8 weights and blockwise FP8 activations go together", name);
  if (block) return MOE_OK;
  if (fp8_act && w->dtype != MOE_DTYPE_FP8_E4M3 && w->dtype != MOE_DTYPE_MXFP4)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: FP8 activations need FP8 or MXFP4 weights", name);
  if (!fp8_act && w->dtype == MOE_DTYPE_FP8_E4M3)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: FP8 weights need FP8 activations", name);
  return MOE_OK;
}

// The GEMMs address each operand through a buffer descriptor with a 32-bit
// byte range: one expert's weights and the permuted rows must each span
// less than 4 GiB.
int check_gemm_extent(int64_t rows, int32_t K, int64_t N_total) {
  const int64_t lim = int64_t(0xFFFFFFFF);
  if (rows * K * 2 > lim) return fail(MOE_ERR_INVALID_ARGUMENT, "permuted rows span more than 4 GiB");
  // (bf16 weights bound MXFP4 ones, which take a quarter of the bytes)
  if (N_total * K * 2 > lim) return fail(MOE_ERR_INVALID_ARGUMENT, "one expert's weights span more than 4 GiB");
  return MOE_OK;
}

int check_rpad(int64_t T, int32_t k, int64_t R_pad) {
  if (R_pad < T * k) return fail(MOE_ERR_SIZE_MISMATCH, "R_pad (%lld) < T * k (%lld)", (long long)R_pad, (long long)(T * k));
  if (R_pad >= (int64_t(1) << 31)) return fail(MOE_ERR_INVALID_ARGUMENT, "R_pad must fit in int32");
  return MOE_OK;
}

struct Carve {
  char* p;
  size_t used = 0;
  template <class T>
  T* take(size_t count) {
    T* r = reinterpret_cast<T*>(p + used);
    used += align_up(count * sizeof(T));
    return r;
  }
};

int check_activation(int32_t activation, float clamp) {
  if (activation != MOE_ACT_SILU && activation != MOE_ACT_GELU)
    return fail(MOE_ERR_UNSUPPORTED, "unknown activation %d", activation);
  if (!(clamp >= 0.0f) || clamp > 3.0e38f)
    return fail(MOE_ERR_INVALID_ARGUMENT, "activation_clamp must be finite and >= 0");
  return MOE_OK;
}

// Options of the fused entry points, checked.
struct LayerOpts {
  int act = MOE_ACT_SILU;
  float clamp = 0.0f;
  bool weight_on_input = false;
  int64_t chunk = 0;  // 0: one pass
  int batch_m = 0;    // > 0: batched experts format with this capacity
  bool fp8 = false;   // FP8 activations (MOE_QUANT_FP8 or MOE_QUANT_FP8X2)
  int terms = 1;      // 2: two-term FP8 activations (MOE_QUANT_FP8X2)
  bool block = false; // blockwise FP8 activations and weights (MOE_QUANT_FP8_BLOCK)
  const float* a1_scale = nullptr;
  const float* a2_scale = nullptr;
};

int parse_options(const moe_layer_options* o, int32_t k, LayerOpts* out) {
  *out = LayerOpts{};
  if (!o) return MOE_OK;
  MOE_CHECK(check_activation(o->activation, o->activation_clamp));
  if (o->apply_router_weight_on_input && k != 1)
    return fail(MOE_ERR_INVALID_ARGUMENT,
                "apply_router_weight_on_input needs top_k = 1 (k=%d)", k);
  if (o->chunk_tokens < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "chunk_tokens must be >= 0");
  out->act = o->activation;
  out->clamp = o->activation_clamp;
  out->weight_on_input = o->apply_router_weight_on_input != 0;
  out->chunk = o->chunk_tokens;
  if (o->batched_max_tokens < 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "batched_max_tokens must be >= 0");
  out->batch_m = o->batched_max_tokens;
  if (o->act_quant != MOE_QUANT_NONE && o->act_quant != MOE_QUANT_FP8 &&
      o->act_quant != MOE_QUANT_FP8X2 && o->act_quant != MOE_QUANT_FP8_BLOCK)
    return fail(MOE_ERR_UNSUPPORTED, "unknown activation quantization %d", o->act_quant);
  out->fp8 = o->act_quant != MOE_QUANT_NONE;
  out->terms = o->act_quant == MOE_QUANT_FP8X2 ? 2 : 1;
  out->block = o->act_quant == MOE_QUANT_FP8_BLOCK;
  if (out->block && (o->a1_scale || o->a2_scale))
    return fail(MOE_ERR_INVALID_ARGUMENT, "blockwise FP8 activations take dynamic scales only");
  if (out->block && out->weight_on_input)
    return fail(MOE_ERR_UNSUPPORTED, "blockwise FP8 activations take no router weight on the input");
  if (out->terms == 2 && (o->a1_scale || o->a2_scale))
    return fail(MOE_ERR_INVALID_ARGUMENT, "two-term FP8 activations take dynamic scales only");
  if (!out->fp8 && (o->a1_scale || o->a2_scale))
    return fail(MOE_ERR_INVALID_ARGUMENT, "a1_scale / a2_scale need act_quant = MOE_QUANT_FP8");
  MOE_CHECK(opt_ptr4(o->a1_scale, "a1_scale"));
  MOE_CHECK(opt_ptr4(o->a2_scale, "a2_scale"));
  out->a1_scale = o->a1_scale;
  out->a2_scale = o->a2_scale;
  return MOE_OK;
}

// Tokens per pass: all T, or the chunk size when it is smaller.
int64_t pass_tokens(int64_t T, const LayerOpts& o) {
  return (o.chunk > 0 && o.chunk < T) ? o.chunk : T;
}

// split-reduction scratch shared by the two routed GEMMs (one after the other)
size_t routed_split_bytes(int64_t R_pad, int32_t H, int32_t I) {
  return std::max(moe::gemm_split_ws_bytes(R_pad, 2 * I), moe::gemm_split_ws_bytes(R_pad, H));
}

// Permuted rows of a pass of T tokens: round_up(T * k, 128), or E_l
// capacity blocks in the batched experts format.
int64_t routed_rows(int64_t T, int32_t k, int32_t E_l, int batch_m) {
  return batch_m > 0 ? int64_t(E_l) * batch_m : moe_permuted_rows(T, k);
}

size_t routed_ws_bytes(int64_t T, int32_t k, int32_t E_l, int32_t H, int32_t I, int batch_m,
                       bool fp8 = false, int terms = 1, bool block = false) {
  // scales per row: one, or one per 128 elements (blockwise)
  const int64_t gh = block ? H / 128 : 1, gi = block ? I / 128 : 1;
  const int64_t R_pad = routed_rows(T, k, E_l, batch_m);
  size_t b = 0;
  b += align_up(sizeof(int32_t) * T * k);               // topk ids
  b += align_up(sizeof(float) * T * k);                 // topk weights
  b += align_up(sizeof(int32_t) * T * k);               // permute map (finalized form)
  b += align_up(sizeof(int32_t) * (E_l + 1));           // offsets
  b += align_up(sizeof(int32_t) * R_pad);               // inverse map (gathered GEMM1 rows)
  b += align_up(sizeof(uint16_t) * R_pad * H);          // x_perm, then GEMM2 output
  b += align_up(sizeof(uint16_t) * R_pad * I);          // h
  b += align_up(routed_split_bytes(R_pad, H, I));       // GEMM split partials
  if (fp8) {
    b += align_up(size_t(T) * H * terms);               // quantized tokens
    b += align_up(sizeof(float) * T * gh);              // their scales
    b += align_up(sizeof(float) * R_pad * gh);          // permuted row scales
    b += align_up(size_t(R_pad) * I * terms);           // quantized hidden rows
    b += align_up(sizeof(float) * R_pad * gi);          // their scales
  }
  return b;
}

// ---- static scratch of moe_fused_experts_unfinalized_noalloc ---------------
// Device memory the library holds on every device it runs on, for callers
// that cannot allocate.  In host code `scratch` is only a stand-in for the
// symbol: its device address comes from hipGetSymbolAddress, once per device
// (each device has its own copy), and only that address is handed to kernels.
constexpr size_t kNoallocScratchBytes = size_t(MOE_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (its device address).
int noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_DEVICE, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || (reinterpret_cast<uintptr_t>(p) % kAlign))
      return fail(MOE_ERR_HIP, "static scratch has no 256-byte aligned device address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported dtype, score function or activation";
    case MOE_ERR_SIZE_MISMATCH: return "size mismatch";
    case MOE_ERR_MISALIGNED: return "misaligned pointer";
    case MOE_ERR_DEVICE: return "pointer is not device memory";
    case MOE_ERR_DESTINATION_CONFLICT: return "destination conflict";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_err; }

int64_t moe_permuted_rows(int64_t T, int32_t k) {
  if (T <= 0 || k <= 0) return 0;
  return (T * k + 127) / 128 * 128;
}

int moe_workspace_size(int64_t T, int32_t k, int32_t E, int32_t E_l, int32_t H, int32_t I,
                       int32_t w_dtype, int32_t shared_I, const moe_layer_options* options,
                       size_t* bytes) {
  g_err[0] = 0;
  MOE_CHECK(check_route_sizes(T, E, k));
  MOE_CHECK(check_local(E, E_l));
  MOE_CHECK(check_gemm_dims(H, I));
  if (w_dtype != MOE_DTYPE_BF16 && w_dtype != MOE_DTYPE_MXFP4 && w_dtype != MOE_DTYPE_FP8_E4M3 &&
      w_dtype != MOE_DTYPE_FP8_BLOCK)
    return fail(MOE_ERR_UNSUPPORTED, "unknown weight dtype %d", w_dtype);
  if (!bytes) return fail(MOE_ERR_INVALID_ARGUMENT, "bytes must not be NULL");
  LayerOpts o;
  MOE_CHECK(parse_options(options, k, &o));
  const int64_t P = pass_tokens(T, o);
  size_t shared_bytes = 0;
  MOE_CHECK(moe_shared_workspace_size(P, H, shared_I, &shared_bytes));
  *bytes = routed_ws_bytes(P, k, E_l, H, I, o.batch_m, o.fp8, o.terms, o.block) + shared_bytes;
  return MOE_OK;
}

int moe_shared_workspace_size(int64_t T, int32_t H, int32_t shared_I, size_t* bytes) {
  g_err[0] = 0;
  if (T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "num_tokens must be non-negative");
  if (!bytes) return fail(MOE_ERR_INVALID_ARGUMENT, "bytes must not be NULL");
  if (shared_I < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "shared_I must be >= 0");
  if (shared_I == 0) {
    *bytes = 0;
    return MOE_OK;
  }
  MOE_CHECK(check_gemm_dims(H, shared_I));
  *bytes = align_up(sizeof(int32_t) * 2) + align_up(sizeof(uint16_t) * T * shared_I) +
           align_up(sizeof(uint16_t) * T * H);
  return MOE_OK;
}

int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t score_fn,
                   int32_t renormalize, float rsf, int32_t* topk_ids, float* topk_weights,
                   void* stream) {
  g_err[0] = 0;
  MOE_CHECK(check_route_sizes(T, E, k));
  if (score_fn != MOE_SCORE_SOFTMAX && score_fn != MOE_SCORE_SIGMOID)
    return fail(MOE_ERR_UNSUPPORTED, "unknown score function %d", score_fn);
  if (T == 0) return MOE_OK;
  MOE_CHECK(need_ptr(logits, "logits"));
  MOE_CHECK(need_ptr(topk_ids, "topk_ids"));
  MOE_CHECK(need_ptr(topk_weights, "topk_weights"));
  hipError_t e = moe::launch_route_topk(logits, T, E, k, score_fn, renormalize, rsf, topk_ids,
                                        topk_weights, nullptr, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route_topk");
}

int moe_permute(const int32_t* topk_ids, const int32_t* expert_map, int64_t T, int32_t k,
                int32_t E, int32_t E_l, const void* x, int32_t H, int64_t R_pad, int32_t* map,
                int32_t* offsets, int32_t* inv, void* x_perm, const float* x_weights,
                void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  (void)workspace;
  (void)workspace_bytes;
  MOE_CHECK(check_route_sizes(T, E, k));
  MOE_CHECK(check_local(E, E_l));
  if (!expert_map && E_l != E)
    return fail(MOE_ERR_INVALID_ARGUMENT, "without an expert map every expert is local (E_l=%d, E=%d)", E_l, E);
  MOE_CHECK(check_rpad(T, k, R_pad));
  if (x_perm && (H <= 0 || H % 8)) return fail(MOE_ERR_INVALID_ARGUMENT, "H must be a positive multiple of 8 (H=%d)", H);
  MOE_CHECK(need_ptr(offsets, "offsets"));
  MOE_CHECK(opt_ptr(inv, "inv"));
  MOE_CHECK(opt_ptr(x_perm, "x_perm"));
  MOE_CHECK(opt_ptr(x_weights, "x_weights"));
  MOE_CHECK(opt_ptr(expert_map, "expert_map"));
  if (T > 0) {
    MOE_CHECK(need_ptr(topk_ids, "topk_ids"));
    MOE_CHECK(need_ptr(map, "map"));
    if (x_perm) MOE_CHECK(need_ptr(x, "x"));
  }
  if (x_perm && overlap(x, sizeof(uint16_t) * T * H, x_perm, sizeof(uint16_t) * R_pad * H))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "x_perm must not overlap x");
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Offsets (and the inverse map's padding) are written even for T = 0.
  hipError_t e = moe::launch_permute(topk_ids, expert_map, T, k, E, E_l, map, offsets, inv, R_pad, s);
  if (e != hipSuccess) return hip_fail(e, "moe_permute");
  if (x_perm && T > 0) {
    e = moe::launch_gather_rows(x, map, T, k, H, x_weights, x_perm, s);
    if (e != hipSuccess) return hip_fail(e, "moe_permute gather");
  }
  return MOE_OK;
}

int moe_route_permute(const float* logits, int64_t T, int32_t E, int32_t k, int32_t score_fn,
                      int32_t renormalize, float rsf, const int32_t* expert_map, int32_t E_l,
                      int64_t R_pad, int32_t* topk_ids, float* topk_weights, int32_t* map,
                      int32_t* offsets, int32_t* inv, void* stream) {
  g_err[0] = 0;
  MOE_CHECK(check_route_sizes(T, E, k));
  if (score_fn != MOE_SCORE_SOFTMAX && score_fn != MOE_SCORE_SIGMOID)
    return fail(MOE_ERR_UNSUPPORTED, "unknown score function %d", score_fn);
  MOE_CHECK(check_local(E, E_l));
  if (!expert_map && E_l != E)
    return fail(MOE_ERR_INVALID_ARGUMENT, "without an expert map every expert is local (E_l=%d, E=%d)", E_l, E);
  MOE_CHECK(check_rpad(T, k, R_pad));
  MOE_CHECK(need_ptr(offsets, "offsets"));
  MOE_CHECK(opt_ptr(inv, "inv"));
  MOE_CHECK(opt_ptr(expert_map, "expert_map"));
  if (T > 0) {
    MOE_CHECK(need_ptr(logits, "logits"));
    MOE_CHECK(need_ptr(topk_ids, "topk_ids"));
    MOE_CHECK(need_ptr(topk_weights, "topk_weights"));
    MOE_CHECK(need_ptr(map, "map"));
  }
  // offsets (and the inverse map's padding) are written even for T = 0
  hipError_t e = moe::launch_route_permute(logits, T, E, k, score_fn, renormalize, rsf, topk_ids,
                                           topk_weights, nullptr, expert_map, E_l, map, offsets,
                                           inv, R_pad, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route_permute");
}

int check_capacity(int32_t E_l, int32_t max_tokens) {
  if (max_tokens <= 0) return fail(MOE_ERR_INVALID_ARGUMENT, "max_tokens must be positive");
  if (int64_t(E_l) * max_tokens >= (int64_t(1) << 31))
    return fail(MOE_ERR_INVALID_ARGUMENT, "E_l * max_tokens must fit in int32");
  return MOE_OK;
}

int moe_permute_batched(const int32_t* topk_ids, const int32_t* expert_map, int64_t T, int32_t k,
                        int32_t E, int32_t E_l, const void* x, int32_t H, int32_t max_tokens,
                        int32_t* map, int32_t* expert_num_tokens, void* x_batched,
                        const float* x_weights, void* stream) {
  g_err[0] = 0;
  MOE_CHECK(check_route_sizes(T, E, k));
  MOE_CHECK(check_local(E, E_l));
  MOE_CHECK(check_capacity(E_l, max_tokens));
  if (!expert_map && E_l != E)
    return fail(MOE_ERR_INVALID_ARGUMENT, "without an expert map every expert is local (E_l=%d, E=%d)", E_l, E);
  if (x_batched && (H <= 0 || H % 8)) return fail(MOE_ERR_INVALID_ARGUMENT, "H must be a positive multiple of 8 (H=%d)", H);
  MOE_CHECK(need_ptr(expert_num_tokens, "expert_num_tokens"));
  MOE_CHECK(opt_ptr(x_batched, "x_batched"));
  MOE_CHECK(opt_ptr(x_weights, "x_weights"));
  MOE_CHECK(opt_ptr(expert_map, "expert_map"));
  if (T > 0) {
    MOE_CHECK(need_ptr(topk_ids, "topk_ids"));
    MOE_CHECK(need_ptr(map, "map"));
    if (x_batched) MOE_CHECK(need_ptr(x, "x"));
  }
  const int64_t rows = int64_t(E_l) * max_tokens;
  if (x_batched && overlap(x, sizeof(uint16_t) * T * H, x_batched, sizeof(uint16_t) * rows * H))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "x_batched must not overlap x");
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the counts are written even for T = 0
  hipError_t e = moe::launch_permute(topk_ids, expert_map, T, k, E, E_l, map, expert_num_tokens,
                                     nullptr, rows, s, max_tokens);
  if (e != hipSuccess) return hip_fail(e, "moe_permute_batched");
  if (x_batched && T > 0) {
    e = moe::launch_gather_rows(x, map, T, k, H, x_weights, x_batched, s);
    if (e != hipSuccess) return hip_fail(e, "moe_permute_batched gather");
  }
  return MOE_OK;
}

// Checks the arguments of one grouped GEMM call and fills *g (R_pad = 0:
// nothing to launch, *g untouched).
static int gemm_check(const void* a, const int32_t* offsets, int32_t E_l, int64_t R_pad,
                      int32_t K, int32_t N_out, int gated, int act, float clamp,
                      const moe_weights* w, void* c, void* workspace, size_t workspace_bytes,
                      const char* name, moe::GemmArgs* g, int batch_m = 0, bool fp8 = false,
                      const float* a_scales = nullptr, int a_terms = 1,
                      const int32_t* a_inv = nullptr, int a_k = 1, int64_t a_T = 0,
                      bool block = false) {
  if (E_l <= 0 || E_l > 1024) return fail(MOE_ERR_INVALID_ARGUMENT, "%s: E_l must be in [1, 1024]", name);
  if (R_pad < 0 || R_pad >= (int64_t(1) << 31)) return fail(MOE_ERR_INVALID_ARGUMENT, "%s: R_pad must be in [0, 2^31)", name);
  MOE_CHECK(check_weights(w, name));
  MOE_CHECK(check_pairing(w, fp8, name, block));
  if (a_terms == 2 && w->dtype != MOE_DTYPE_MXFP4)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: two-term FP8 activations need MXFP4 weights", name);
  // (two-term rows take 2K bytes, as many as bf16 rows)
  MOE_CHECK(check_gemm_extent(R_pad, K, gated ? 2 * int64_t(N_out) : N_out));
  if (R_pad == 0) return MOE_OK;
  MOE_CHECK(need_ptr(a, "input rows"));
  MOE_CHECK(need_ptr(offsets, "offsets"));
  MOE_CHECK(need_ptr(c, "output rows"));
  // (gathered: the token rows, at most R_pad of them)
  const size_t in_bytes = (fp8 ? a_terms : sizeof(uint16_t)) * (a_inv ? a_T : R_pad) * K;
  const size_t out_bytes = sizeof(uint16_t) * R_pad * N_out;
  if (overlap(a, in_bytes, c, out_bytes))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "%s: output must not overlap the input rows", name);
  const size_t scale_bytes = sizeof(float) * R_pad * (block ? K / 128 : 1);
  if (a_scales && overlap(a_scales, scale_bytes, c, out_bytes))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "%s: output must not overlap the row scales", name);
  if (workspace_bytes > 0) {
    MOE_CHECK(need_ptr(workspace, "workspace"));
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
      return fail(MOE_ERR_MISALIGNED, "%s: workspace must be 256-byte aligned", name);
    if (overlap(workspace, workspace_bytes, a, in_bytes) || overlap(workspace, workspace_bytes, c, out_bytes))
      return fail(MOE_ERR_DESTINATION_CONFLICT, "%s: workspace must not overlap the rows", name);
  }
  *g = moe::GemmArgs{a, w->data, scales_of(w), offsets, E_l, K, N_out, gated, R_pad, c,
                     workspace_bytes > 0 ? workspace : nullptr, workspace_bytes, act, clamp,
                     batch_m, a_scales, w->dtype == MOE_DTYPE_MXFP4, a_terms, a_inv, a_k, a_T};
  if (block) g->a_ld = R_pad;
  return MOE_OK;
}

static int gemm_common(const void* a, const int32_t* offsets, int32_t E_l, int64_t R_pad,
                       int32_t K, int32_t N_out, int gated, int act, float clamp,
                       const moe_weights* w, void* c, void* workspace, size_t workspace_bytes,
                       void* stream, const char* name, int batch_m = 0, int64_t max_rows = 0,
                       bool fp8 = false, const float* a_scales = nullptr, int a_terms = 1,
                       const int32_t* a_inv = nullptr, int a_k = 1, int64_t a_T = 0,
                       bool block = false) {
  moe::GemmArgs g{};
  MOE_CHECK(gemm_check(a, offsets, E_l, R_pad, K, N_out, gated, act, clamp, w, c, workspace,
                       workspace_bytes, name, &g, batch_m, fp8, a_scales, a_terms, a_inv, a_k,
                       a_T, block));
  if (R_pad == 0) return MOE_OK;
  const int64_t rows_bound = (max_rows > 0 && max_rows < R_pad) ? max_rows : R_pad;
  hipError_t e = moe::launch_grouped_gemm(g, rows_bound, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, name);
}

int moe_grouped_gemm1_act(const void* a_perm, const int32_t* offsets, int32_t E_l, int64_t R_pad,
                          int32_t H, int32_t I, const moe_weights* w1, int32_t activation,
                          float activation_clamp, void* h, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  MOE_CHECK(check_gemm_dims(H, I));
  MOE_CHECK(check_activation(activation, activation_clamp));
  return gemm_common(a_perm, offsets, E_l, R_pad, H, I, 1, activation, activation_clamp, w1, h,
                     workspace, workspace_bytes, stream, "moe_grouped_gemm1_act");
}

int moe_grouped_gemm1_act_gathered(const void* x, const int32_t* inv, int64_t T, int32_t k,
                                   const int32_t* offsets, int32_t E_l, int64_t R_pad, int32_t H,
                                   int32_t I, const moe_weights* w1, int32_t activation,
                                   float activation_clamp, void* h, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  MOE_CHECK(check_gemm_dims(H, I));
  MOE_CHECK(check_activation(activation, activation_clamp));
  if (T < 0 || k <= 0) return fail(MOE_ERR_INVALID_ARGUMENT, "T must be >= 0 and k > 0");
  if (R_pad < T * k) return fail(MOE_ERR_SIZE_MISMATCH, "R_pad (%lld) < T * k (%lld)",
                                 (long long)R_pad, (long long)(T * k));
  if (T * int64_t(H) * 2 > int64_t(0xFFFFFFFF))
    return fail(MOE_ERR_INVALID_ARGUMENT, "x spans more than 4 GiB");
  if (R_pad > 0) MOE_CHECK(need_ptr(inv, "inv"));
  if (overlap(inv, sizeof(int32_t) * R_pad, h, sizeof(uint16_t) * R_pad * I))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "h must not overlap inv");
  if (R_pad == 0 || T == 0) {
    MOE_CHECK(check_weights(w1, "moe_grouped_gemm1_act_gathered"));
    return MOE_OK;
  }
  return gemm_common(x, offsets, E_l, R_pad, H, I, 1, activation, activation_clamp, w1, h,
                     workspace, workspace_bytes, stream, "moe_grouped_gemm1_act_gathered", 0, 0,
                     false, nullptr, 1, inv, k, T);
}

int moe_route_permute_gemm1_act(const float* logits, const void* x, int64_t T, int32_t H,
                                int32_t I, int32_t E, int32_t E_l, int32_t k, int32_t score_fn,
                                int32_t renormalize, float rsf, const int32_t* expert_map,
                                int64_t R_pad, const moe_weights* w1, int32_t activation,
                                float activation_clamp, int32_t* topk_ids, float* topk_weights,
                                int32_t* map, int32_t* offsets, int32_t* inv, void* h,
                                void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  MOE_CHECK(check_route_sizes(T, E, k));
  if (score_fn != MOE_SCORE_SOFTMAX && score_fn != MOE_SCORE_SIGMOID)
    return fail(MOE_ERR_UNSUPPORTED, "unknown score function %d", score_fn);
  MOE_CHECK(check_local(E, E_l));
  if (!expert_map && E_l != E)
    return fail(MOE_ERR_INVALID_ARGUMENT, "without an expert map every expert is local (E_l=%d, E=%d)", E_l, E);
  MOE_CHECK(check_rpad(T, k, R_pad));
  MOE_CHECK(check_gemm_dims(H, I));
  MOE_CHECK(check_activation(activation, activation_clamp));
  if (T * int64_t(H) * 2 > int64_t(0xFFFFFFFF))
    return fail(MOE_ERR_INVALID_ARGUMENT, "x spans more than 4 GiB");
  MOE_CHECK(need_ptr(offsets, "offsets"));
  MOE_CHECK(opt_ptr(expert_map, "expert_map"));
  if (R_pad > 0) MOE_CHECK(need_ptr(inv, "inv"));
  if (T > 0) {
    MOE_CHECK(need_ptr(logits, "logits"));
    MOE_CHECK(need_ptr(topk_ids, "topk_ids"));
    MOE_CHECK(need_ptr(topk_weights, "topk_weights"));
    MOE_CHECK(need_ptr(map, "map"));
  }
  if (overlap(inv, sizeof(int32_t) * R_pad, h, sizeof(uint16_t) * R_pad * I))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "h must not overlap inv");
  moe::GemmArgs g{};
  MOE_CHECK(gemm_check(x, offsets, E_l, R_pad, H, I, 1, activation, activation_clamp, w1, h,
                       workspace, workspace_bytes, "moe_route_permute_gemm1_act", &g, 0, false,
                       nullptr, 1, inv, k, T));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T > 0 && R_pad > 0 && moe::gemm_picks_decode(g, R_pad) &&
      moe::decode_route_gemm1_fits(g, T, E, k)) {
    hipError_t e = moe::launch_decode_route_gemm1(logits, T, E, k, score_fn, renormalize, rsf,
                                                  topk_ids, topk_weights, nullptr, expert_map,
                                                  map, offsets, inv, R_pad, g, s);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route_permute_gemm1_act");
  }
  // offsets (and the inverse map's padding) are written even for T = 0
  hipError_t e = moe::launch_route_permute(logits, T, E, k, score_fn, renormalize, rsf, topk_ids,
                                           topk_weights, nullptr, expert_map, E_l, map, offsets,
                                           inv, R_pad, 0, s);
  if (e != hipSuccess) return hip_fail(e, "moe_route_permute_gemm1_act route");
  if (T == 0 || R_pad == 0) return MOE_OK;
  e = moe::launch_grouped_gemm(g, R_pad, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route_permute_gemm1_act gemm1");
}

int moe_grouped_gemm2(const void* h, const int32_t* offsets, int32_t E_l, int64_t R_pad,
                      int32_t I, int32_t H, const moe_weights* w2, void* y, void* workspace,
                      size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  MOE_CHECK(check_gemm_dims(H, I));
  return gemm_common(h, offsets, E_l, R_pad, I, H, 0, MOE_ACT_SILU, 0.0f, w2, y, workspace,
                     workspace_bytes, stream, "moe_grouped_gemm2");
}

int moe_quantize_fp8(const void* x, int64_t rows, int32_t H, const float* static_scale,
                     const float* row_weights, const int32_t* row_count, uint8_t* q,
                     float* scales, void* stream) {
  g_err[0] = 0;
  if (rows < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "rows must be non-negative");
  if (H <= 0 || H % 16) return fail(MOE_ERR_INVALID_ARGUMENT, "H must be a positive multiple of 16 (H=%d)", H);
  if (rows == 0) return MOE_OK;
  MOE_CHECK(need_ptr(x, "x"));
  MOE_CHECK(need_ptr(q, "q"));
  MOE_CHECK(need_ptr(scales, "scales"));
  MOE_CHECK(opt_ptr4(static_scale, "static_scale"));
  MOE_CHECK(opt_ptr4(row_weights, "row_weights"));
  MOE_CHECK(opt_ptr4(row_count, "row_count"));
  if (overlap(x, sizeof(uint16_t) * rows * H, q, size_t(rows) * H) ||
      overlap(x, sizeof(uint16_t) * rows * H, scales, sizeof(float) * rows))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "q and scales must not overlap x");
  hipError_t e = moe::launch_quantize_fp8(x, rows, H, static_scale, row_weights, row_count, q,
                                          scales, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_quantize_fp8");
}

int moe_permute_fp8(const int32_t* topk_ids, const int32_t* expert_map, int64_t T, int32_t k,
                    int32_t E, int32_t E_l, const uint8_t* xq, const float* x_scales, int32_t H,
                    int64_t R_pad, int32_t* map, int32_t* offsets, int32_t* inv, uint8_t* xq_perm,
                    float* xq_perm_scales, void* stream) {
  g_err[0] = 0;
  MOE_CHECK(check_route_sizes(T, E, k));
  MOE_CHECK(check_local(E, E_l));
  if (!expert_map && E_l != E)
    return fail(MOE_ERR_INVALID_ARGUMENT, "without an expert map every expert is local (E_l=%d, E=%d)", E_l, E);
  MOE_CHECK(check_rpad(T, k, R_pad));
  if (H <= 0 || H % 16) return fail(MOE_ERR_INVALID_ARGUMENT, "H must be a positive multiple of 16 (H=%d)", H);
  MOE_CHECK(need_ptr(offsets, "offsets"));
  MOE_CHECK(opt_ptr(inv, "inv"));
  MOE_CHECK(opt_ptr(expert_map, "expert_map"));
  if (T > 0) {
    MOE_CHECK(need_ptr(topk_ids, "topk_ids"));
    MOE_CHECK(need_ptr(map, "map"));
    MOE_CHECK(need_ptr(xq, "xq"));
    MOE_CHECK(need_ptr(xq_perm, "xq_perm"));
    MOE_CHECK(opt_ptr4(x_scales, "x_scales"));
    MOE_CHECK(opt_ptr4(xq_perm_scales, "xq_perm_scales"));
    if (!x_scales || !xq_perm_scales)
      return fail(MOE_ERR_INVALID_ARGUMENT, "x_scales and xq_perm_scales must not be NULL");
  }
  if (overlap(xq, size_t(T) * H, xq_perm, size_t(R_pad) * H))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "xq_perm must not overlap xq");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = moe::launch_permute(topk_ids, expert_map, T, k, E, E_l, map, offsets, inv, R_pad, s);
  if (e != hipSuccess) return hip_fail(e, "moe_permute_fp8");
  if (T > 0) {
    e = moe::launch_gather_fp8_rows(xq, x_scales, map, T, k, H, xq_perm, xq_perm_scales, s);
    if (e != hipSuccess) return hip_fail(e, "moe_permute_fp8 gather");
  }
  return MOE_OK;
}

// FP8 activations: k-steps of 128; with MXFP4 weights, weight stages of 256
// (one 8-byte load of E8M0 scales per row and stage)
int check_fp8_dims(int32_t H, int32_t I, const moe_weights* w = nullptr) {
  const int q = (w && w->dtype == MOE_DTYPE_MXFP4) ? 256 : 128;
  if (H % q || I % q)
    return fail(MOE_ERR_INVALID_ARGUMENT, "FP8 GEMMs need H and I multiples of %d (H=%d, I=%d)",
                q, H, I);
  return MOE_OK;
}

int moe_grouped_gemm1_act_fp8(const uint8_t* a_perm, const float* a_scales,
                              const int32_t* offsets, int32_t E_l, int64_t R_pad, int32_t H,
                              int32_t I, const moe_weights* w1, int32_t activation,
                              float activation_clamp, void* h, void* workspace,
                              size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  MOE_CHECK(check_gemm_dims(H, I));
  MOE_CHECK(check_fp8_dims(H, I, w1));
  MOE_CHECK(check_activation(activation, activation_clamp));
  if (R_pad > 0) MOE_CHECK(opt_ptr4(a_scales, "a_scales"));
  if (R_pad > 0 && !a_scales) return fail(MOE_ERR_INVALID_ARGUMENT, "a_scales must not be NULL");
  return gemm_common(a_perm, offsets, E_l, R_pad, H, I, 1, activation, activation_clamp, w1, h,
                     workspace, workspace_bytes, stream, "moe_grouped_gemm1_act_fp8", 0, 0, true,
                     a_scales);
}

int moe_grouped_gemm2_fp8(const uint8_t* h_perm, const float* h_scales, const int32_t* offsets,
                          int32_t E_l, int64_t R_pad, int32_t I, int32_t H, const moe_weights* w2,
                          void* y, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  MOE_CHECK(check_gemm_dims(H, I));
  MOE_CHECK(check_fp8_dims(H, I, w2));
  if (R_pad > 0) MOE_CHECK(opt_ptr4(h_scales, "h_scales"));
  if (R_pad > 0 && !h_scales) return fail(MOE_ERR_INVALID_ARGUMENT, "h_scales must not be NULL");
  return gemm_common(h_perm, offsets, E_l, R_pad, I, H, 0, MOE_ACT_SILU, 0.0f, w2, y, workspace,
                     workspace_bytes, stream, "moe_grouped_gemm2_fp8", 0, 0, true, h_scales);
}

int moe_grouped_gemm1_act_fp8_gathered(const uint8_t* xq, const float* x_scales,
                                       int32_t terms, const int32_t* inv, int64_t T, int32_t k,
                                       const int32_t* offsets, int32_t E_l, int64_t R_pad,
                                       int32_t H, int32_t I, const moe_weights* w1,
                                       int32_t activation, float activation_clamp, void* h,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  MOE_CHECK(check_gemm_dims(H, I));
  MOE_CHECK(check_fp8_dims(H, I, w1));
  MOE_CHECK(check_activation(activation, activation_clamp));
  if (terms != 1 && terms != 2) return fail(MOE_ERR_INVALID_ARGUMENT, "terms must be 1 or 2");
  if (T < 0 || k <= 0) return fail(MOE_ERR_INVALID_ARGUMENT, "T must be >= 0 and k > 0");
  if (R_pad < T * k) return fail(MOE_ERR_SIZE_MISMATCH, "R_pad (%lld) < T * k (%lld)",
                                 (long long)R_pad, (long long)(T * k));
  if (T * int64_t(H) * terms > int64_t(0xFFFFFFFF))
    return fail(MOE_ERR_INVALID_ARGUMENT, "xq spans more than 4 GiB");
  if (R_pad > 0) MOE_CHECK(need_ptr(inv, "inv"));
  if (overlap(inv, sizeof(int32_t) * R_pad, h, sizeof(uint16_t) * R_pad * I))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "h must not overlap inv");
  if (R_pad == 0 || T == 0) {
    MOE_CHECK(check_weights(w1, "moe_grouped_gemm1_act_fp8_gathered"));
    return MOE_OK;
  }
  MOE_CHECK(opt_ptr4(x_scales, "x_scales"));
  if (!x_scales) return fail(MOE_ERR_INVALID_ARGUMENT, "x_scales must not be NULL");
  return gemm_common(xq, offsets, E_l, R_pad, H, I, 1, activation, activation_clamp, w1, h,
                     workspace, workspace_bytes, stream, "moe_grouped_gemm1_act_fp8_gathered", 0,
                     0, true, x_scales, terms, inv, k, T);
}

int moe_quantize_fp8_blockwise(const void* x, int64_t rows, int32_t H, const int32_t* row_count,
                               uint8_t* q, float* scales, int64_t scales_ld, void* stream) {
  g_err[0] = 0;
  if (rows < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "rows must be non-negative");
  if (H <= 0 || H % 128)
    return fail(MOE_ERR_INVALID_ARGUMENT, "H must be a positive multiple of 128 (H=%d)", H);
  if (scales_ld < rows) return fail(MOE_ERR_SIZE_MISMATCH, "scales_ld must be >= rows");
  if (rows == 0) return MOE_OK;
  MOE_CHECK(need_ptr(x, "x"));
  MOE_CHECK(need_ptr(q, "q"));
  MOE_CHECK(need_ptr(scales, "scales"));
  MOE_CHECK(opt_ptr4(row_count, "row_count"));
  const size_t sc_bytes = sizeof(float) * size_t(scales_ld) * (H / 128);
  if (overlap(x, sizeof(uint16_t) * rows * H, q, size_t(rows) * H) ||
      overlap(x, sizeof(uint16_t) * rows * H, scales, sc_bytes) ||
      overlap(q, size_t(rows) * H, scales, sc_bytes))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "x, q and scales must not overlap");
  hipError_t e = moe::launch_quantize_fp8_groups(x, rows, H, row_count, q, scales, scales_ld,
                                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_quantize_fp8_blockwise");
}

int moe_permute_fp8_blockwise(const int32_t* topk_ids, const int32_t* expert_map, int64_t T,
                              int32_t k, int32_t E, int32_t E_l, const uint8_t* xq,
                              const float* x_scales, int32_t H, int64_t R_pad, int32_t* map,
                              int32_t* offsets, int32_t* inv, uint8_t* xq_perm,
                              float* xq_perm_scales, void* stream) {
  g_err[0] = 0;
  MOE_CHECK(check_route_sizes(T, E, k));
  MOE_CHECK(check_local(E, E_l));
  if (!expert_map && E_l != E)
    return fail(MOE_ERR_INVALID_ARGUMENT, "without an expert map every expert is local (E_l=%d, E=%d)", E_l, E);
  MOE_CHECK(check_rpad(T, k, R_pad));
  if (H <= 0 || H % 128)
    return fail(MOE_ERR_INVALID_ARGUMENT, "H must be a positive multiple of 128 (H=%d)", H);
  MOE_CHECK(need_ptr(offsets, "offsets"));
  MOE_CHECK(opt_ptr(inv, "inv"));
  MOE_CHECK(opt_ptr(expert_map, "expert_map"));
  if (T > 0) {
    MOE_CHECK(need_ptr(topk_ids, "topk_ids"));
    MOE_CHECK(need_ptr(map, "map"));
    MOE_CHECK(need_ptr(xq, "xq"));
    MOE_CHECK(need_ptr(xq_perm, "xq_perm"));
    MOE_CHECK(opt_ptr4(x_scales, "x_scales"));
    MOE_CHECK(opt_ptr4(xq_perm_scales, "xq_perm_scales"));
    if (!x_scales || !xq_perm_scales)
      return fail(MOE_ERR_INVALID_ARGUMENT, "x_scales and xq_perm_scales must not be NULL");
  }
  if (overlap(xq, size_t(T) * H, xq_perm, size_t(R_pad) * H) ||
      overlap(x_scales, sizeof(float) * T * (H / 128), xq_perm_scales,
              sizeof(float) * R_pad * (H / 128)))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "xq_perm and its scales must not overlap xq and its scales");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = moe::launch_permute(topk_ids, expert_map, T, k, E, E_l, map, offsets, inv, R_pad, s);
  if (e != hipSuccess) return hip_fail(e, "moe_permute_fp8_blockwise");
  if (T > 0) {
    e = moe::launch_gather_fp8_rows(xq, x_scales, map, T, k, H, xq_perm, xq_perm_scales, s,
                                    H / 128, R_pad);
    if (e != hipSuccess) return hip_fail(e, "moe_permute_fp8_blockwise gather");
  }
  return MOE_OK;
}

int moe_grouped_gemm1_act_fp8_blockwise(const uint8_t* a_perm, const float* a_scales,
                                        const int32_t* offsets, int32_t E_l, int64_t R_pad,
                                        int32_t H, int32_t I, const moe_weights* w1,
                                        int32_t activation, float activation_clamp, void* h,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  MOE_CHECK(check_gemm_dims(H, I));
  MOE_CHECK(check_fp8_dims(H, I, w1));
  MOE_CHECK(check_activation(activation, activation_clamp));
  if (R_pad > 0) MOE_CHECK(opt_ptr4(a_scales, "a_scales"));
  if (R_pad > 0 && !a_scales) return fail(MOE_ERR_INVALID_ARGUMENT, "a_scales must not be NULL");
  return gemm_common(a_perm, offsets, E_l, R_pad, H, I, 1, activation, activation_clamp, w1, h,
                     workspace, workspace_bytes, stream, "moe_grouped_gemm1_act_fp8_blockwise", 0,
                     0, true, a_scales, 1, nullptr, 1, 0, true);
}

int moe_grouped_gemm2_fp8_blockwise(const uint8_t* h_perm, const float* h_scales,
                                    const int32_t* offsets, int32_t E_l, int64_t R_pad,
                                    int32_t I, int32_t H, const moe_weights* w2, void* y,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  MOE_CHECK(check_gemm_dims(H, I));
  MOE_CHECK(check_fp8_dims(H, I, w2));
  if (R_pad > 0) MOE_CHECK(opt_ptr4(h_scales, "h_scales"));
  if (R_pad > 0 && !h_scales) return fail(MOE_ERR_INVALID_ARGUMENT, "h_scales must not be NULL");
  return gemm_common(h_perm, offsets, E_l, R_pad, I, H, 0, MOE_ACT_SILU, 0.0f, w2, y, workspace,
                     workspace_bytes, stream, "moe_grouped_gemm2_fp8_blockwise", 0, 0, true,
                     h_scales, 1, nullptr, 1, 0, true);
}

int moe_quantize_fp8x2(const void* x, int64_t rows, int32_t H, const float* row_weights,
                       const int32_t* row_count, uint8_t* q, float* scales, void* stream) {
  g_err[0] = 0;
  if (rows < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "rows must be non-negative");
  if (H <= 0 || H % 64) return fail(MOE_ERR_INVALID_ARGUMENT, "H must be a positive multiple of 64 (H=%d)", H);
  if (rows == 0) return MOE_OK;
  MOE_CHECK(need_ptr(x, "x"));
  MOE_CHECK(need_ptr(q, "q"));
  MOE_CHECK(need_ptr(scales, "scales"));
  MOE_CHECK(opt_ptr4(row_weights, "row_weights"));
  MOE_CHECK(opt_ptr4(row_count, "row_count"));
  if (overlap(x, sizeof(uint16_t) * rows * H, q, size_t(rows) * H * 2) ||
      overlap(x, sizeof(uint16_t) * rows * H, scales, sizeof(float) * rows))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "q and scales must not overlap x");
  hipError_t e = moe::launch_quantize_fp8(x, rows, H, nullptr, row_weights, row_count, q, scales,
                                          static_cast<hipStream_t>(stream), 2);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_quantize_fp8x2");
}

int moe_grouped_gemm1_act_fp8x2(const uint8_t* a_perm, const float* a_scales,
                                const int32_t* offsets, int32_t E_l, int64_t R_pad, int32_t H,
                                int32_t I, const moe_weights* w1, int32_t activation,
                                float activation_clamp, void* h, void* workspace,
                                size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  MOE_CHECK(check_gemm_dims(H, I));
  MOE_CHECK(check_fp8_dims(H, I, w1));
  MOE_CHECK(check_activation(activation, activation_clamp));
  if (R_pad > 0) MOE_CHECK(opt_ptr4(a_scales, "a_scales"));
  if (R_pad > 0 && !a_scales) return fail(MOE_ERR_INVALID_ARGUMENT, "a_scales must not be NULL");
  return gemm_common(a_perm, offsets, E_l, R_pad, H, I, 1, activation, activation_clamp, w1, h,
                     workspace, workspace_bytes, stream, "moe_grouped_gemm1_act_fp8x2", 0, 0,
                     true, a_scales, 2);
}

int moe_grouped_gemm2_fp8x2(const uint8_t* h_perm, const float* h_scales,
                            const int32_t* offsets, int32_t E_l, int64_t R_pad, int32_t I,
                            int32_t H, const moe_weights* w2, void* y, void* workspace,
                            size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  MOE_CHECK(check_gemm_dims(H, I));
  MOE_CHECK(check_fp8_dims(H, I, w2));
  if (R_pad > 0) MOE_CHECK(opt_ptr4(h_scales, "h_scales"));
  if (R_pad > 0 && !h_scales) return fail(MOE_ERR_INVALID_ARGUMENT, "h_scales must not be NULL");
  return gemm_common(h_perm, offsets, E_l, R_pad, I, H, 0, MOE_ACT_SILU, 0.0f, w2, y, workspace,
                     workspace_bytes, stream, "moe_grouped_gemm2_fp8x2", 0, 0, true, h_scales, 2);
}

int moe_grouped_gemm1_act_batched(const void* a_batched, const int32_t* expert_num_tokens,
                                  int32_t E_l, int32_t max_tokens, int64_t max_rows, int32_t H,
                                  int32_t I, const moe_weights* w1, int32_t activation,
                                  float activation_clamp, void* h_batched, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  MOE_CHECK(check_gemm_dims(H, I));
  MOE_CHECK(check_activation(activation, activation_clamp));
  if (E_l <= 0 || E_l > 1024) return fail(MOE_ERR_INVALID_ARGUMENT, "E_l must be in [1, 1024]");
  MOE_CHECK(check_capacity(E_l, max_tokens));
  if (max_rows < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "max_rows must be >= 0");
  return gemm_common(a_batched, expert_num_tokens, E_l, int64_t(E_l) * max_tokens, H, I, 1,
                     activation, activation_clamp, w1, h_batched, workspace, workspace_bytes,
                     stream, "moe_grouped_gemm1_act_batched", max_tokens, max_rows);
}

int moe_grouped_gemm2_batched(const void* h_batched, const int32_t* expert_num_tokens,
                              int32_t E_l, int32_t max_tokens, int64_t max_rows, int32_t I,
                              int32_t H, const moe_weights* w2, void* y_batched, void* workspace,
                              size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  MOE_CHECK(check_gemm_dims(H, I));
  if (E_l <= 0 || E_l > 1024) return fail(MOE_ERR_INVALID_ARGUMENT, "E_l must be in [1, 1024]");
  MOE_CHECK(check_capacity(E_l, max_tokens));
  if (max_rows < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "max_rows must be >= 0");
  return gemm_common(h_batched, expert_num_tokens, E_l, int64_t(E_l) * max_tokens, I, H, 0,
                     MOE_ACT_SILU, 0.0f, w2, y_batched, workspace, workspace_bytes, stream,
                     "moe_grouped_gemm2_batched", max_tokens, max_rows);
}

int moe_grouped_gemm_workspace_size(int64_t R_pad, int32_t N_out, int32_t gated, size_t* bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(MOE_ERR_INVALID_ARGUMENT, "bytes must not be NULL");
  if (R_pad < 0 || R_pad >= (int64_t(1) << 31))
    return fail(MOE_ERR_INVALID_ARGUMENT, "R_pad must be in [0, 2^31)");
  if (N_out <= 0 || N_out % 64)
    return fail(MOE_ERR_INVALID_ARGUMENT, "N_out must be a positive multiple of 64 (N_out=%d)", N_out);
  *bytes = moe::gemm_split_ws_bytes(R_pad, gated ? 2 * N_out : N_out);
  return MOE_OK;
}

// The rows of gemm2_permuted: non-negative, and their bytes within int64.
int check_y_rows(int64_t y_rows, int32_t H) {
  if (y_rows < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "y_rows must be non-negative (y_rows=%lld)", (long long)y_rows);
  if (y_rows > (int64_t(1) << 62) / (2 * int64_t(H)))
    return fail(MOE_ERR_INVALID_ARGUMENT, "gemm2_permuted is too large (y_rows=%lld)", (long long)y_rows);
  return MOE_OK;
}

int moe_finalize(const void* y_perm, int64_t y_rows, const void* weights, int32_t weights_dtype,
                 const int32_t* map, int64_t T, int32_t k, int32_t H, float rsf_fin,
                 const void* shared, void* out, void* stream) {
  g_err[0] = 0;
  if (T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "num_tokens must be non-negative (T=%lld)", (long long)T);
  if (k <= 0 || k > 32) return fail(MOE_ERR_INVALID_ARGUMENT, "top_k must be in [1, 32] (k=%d)", k);
  if (H <= 0 || H % 8) return fail(MOE_ERR_INVALID_ARGUMENT, "H must be a positive multiple of 8 (H=%d)", H);
  MOE_CHECK(check_y_rows(y_rows, H));
  if (weights_dtype != MOE_DTYPE_F32 && weights_dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "weights must be float32 or bfloat16 (dtype %d)", weights_dtype);
  if (T == 0) return MOE_OK;
  if (y_rows > 0) MOE_CHECK(need_ptr(y_perm, "gemm2_permuted"));
  MOE_CHECK(opt_ptr(weights, "expert_weights"));
  MOE_CHECK(need_ptr(map, "map"));
  MOE_CHECK(opt_ptr(shared, "shared"));
  MOE_CHECK(need_ptr(out, "out"));
  const size_t out_bytes = sizeof(uint16_t) * T * H;
  if (shared && shared != out && overlap(shared, out_bytes, out, out_bytes))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "out must alias shared exactly or not overlap it");
  // every row the kernel may read: map entries past y_rows count as -1
  if (overlap(y_perm, sizeof(uint16_t) * y_rows * H, out, out_bytes))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "out must not overlap gemm2_permuted");
  hipError_t e = moe::launch_finalize(y_perm, y_rows, weights, weights_dtype == MOE_DTYPE_BF16, map,
                                      T, k, H, rsf_fin, shared, out,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_finalize");
}

int moe_finalize_add_rmsnorm(const void* y_perm, int64_t y_rows, const void* weights,
                             int32_t weights_dtype,
                             const int32_t* map, int64_t T, int32_t k, int32_t H, float rsf_fin,
                             const void* shared, void* residual, const void* gamma, float eps,
                             void* out, void* stream) {
  g_err[0] = 0;
  if (T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "num_tokens must be non-negative (T=%lld)", (long long)T);
  if (k <= 0 || k > 32) return fail(MOE_ERR_INVALID_ARGUMENT, "top_k must be in [1, 32] (k=%d)", k);
  if (H <= 0 || H % 8 || H > moe::kTailMaxH)
    return fail(MOE_ERR_INVALID_ARGUMENT, "H must be a positive multiple of 8, at most %d (H=%d)",
                moe::kTailMaxH, H);
  if (!(eps >= 0.0f)) return fail(MOE_ERR_INVALID_ARGUMENT, "eps must be >= 0");
  MOE_CHECK(check_y_rows(y_rows, H));
  if (weights_dtype != MOE_DTYPE_F32 && weights_dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "weights must be float32 or bfloat16 (dtype %d)", weights_dtype);
  if (T == 0) return MOE_OK;
  if (y_rows > 0) MOE_CHECK(need_ptr(y_perm, "gemm2_permuted"));
  MOE_CHECK(opt_ptr(weights, "expert_weights"));
  MOE_CHECK(need_ptr(map, "map"));
  MOE_CHECK(opt_ptr(shared, "shared"));
  MOE_CHECK(need_ptr(residual, "residual"));
  MOE_CHECK(need_ptr(gamma, "gamma"));
  MOE_CHECK(need_ptr(out, "out"));
  const size_t row_bytes = sizeof(uint16_t) * T * H;
  if (overlap(out, row_bytes, residual, row_bytes))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "out must not overlap residual");
  if (shared && overlap(shared, row_bytes, residual, row_bytes))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "shared must not overlap residual (written in place)");
  if (shared && overlap(shared, row_bytes, out, row_bytes))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "out must not overlap shared");
  const size_t y_bytes = sizeof(uint16_t) * y_rows * H;
  if (overlap(y_perm, y_bytes, out, row_bytes) || overlap(y_perm, y_bytes, residual, row_bytes))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "out and residual must not overlap gemm2_permuted");
  hipError_t e = moe::launch_finalize_add_rmsnorm(y_perm, y_rows, weights,
                                                  weights_dtype == MOE_DTYPE_BF16,
                                                  map, T, k, H, rsf_fin, shared, residual, gamma,
                                                  eps, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_finalize_add_rmsnorm");
}

// Workspace of the routed part of the fused entry points (rows sized for
// moe_permuted_rows(T, k), or E_l capacity blocks in the batched experts
// format; the GEMMs never touch rows past the local routes).
struct RoutedWs {
  int32_t* ids;
  float* wts;
  int32_t* map;
  int32_t* offsets;
  int32_t* inv;      // permuted row -> expanded index (GEMM1 reading token rows itself)
  uint16_t* x_perm;  // gathered rows, later reused for the GEMM2 output
  uint16_t* h;
  void* split;       // split-reduction scratch of both GEMMs
  size_t split_bytes;
  int64_t rows;
  // FP8 activations: quantized tokens and scales, permuted row scales (the
  // quantized permuted rows sit in x_perm's slot), quantized hidden rows
  uint8_t* xq = nullptr;
  float* xs = nullptr;
  float* ps = nullptr;
  uint8_t* hq = nullptr;
  float* hs = nullptr;
};

static RoutedWs carve_routed(Carve& c, int64_t T, int32_t k, int32_t E_l, int32_t H, int32_t I,
                             int batch_m, bool fp8 = false, int terms = 1,
                             size_t split_cap = ~size_t(0), bool block = false) {
  const int64_t gh = block ? H / 128 : 1, gi = block ? I / 128 : 1;  // scales per row
  RoutedWs b;
  b.rows = routed_rows(T, k, E_l, batch_m);
  b.ids = c.take<int32_t>(T * k);
  b.wts = c.take<float>(T * k);
  b.map = c.take<int32_t>(T * k);
  b.offsets = c.take<int32_t>(E_l + 1);  // offsets, or per-expert counts when batched
  b.inv = c.take<int32_t>(b.rows);
  b.x_perm = c.take<uint16_t>(b.rows * H);
  b.h = c.take<uint16_t>(b.rows * I);
  // (a smaller split scratch only lowers the number of pieces the GEMMs use)
  b.split_bytes = std::min(routed_split_bytes(b.rows, H, I), split_cap);
  b.split = b.split_bytes ? c.take<char>(b.split_bytes) : nullptr;
  if (fp8) {
    // (two-term quantized permuted rows, 2H bytes each, fill x_perm's slot)
    b.xq = c.take<uint8_t>(T * H * terms);
    b.xs = c.take<float>(T * gh);
    b.ps = c.take<float>(b.rows * gh);
    b.hq = c.take<uint8_t>(b.rows * I * terms);
    b.hs = c.take<float>(b.rows * gi);
  }
  return b;
}

// One-term FP8 batches up to this many tokens read their rows inside GEMM1.
constexpr int64_t kGatherFp8MaxT = 64;

// Route, permute, GEMM1, GEMM2 of T tokens on one stream.  map_out / y_out
// default to the workspace copies; w_bf16_out, when given, receives the bf16
// routing weights (exactly 1 when they go on the inputs).
static int run_routed(const float* logits, const void* x, int64_t T, int32_t H, int32_t I,
                      int32_t E, int32_t E_l, int32_t k, int32_t score_fn, int32_t renormalize,
                      float rsf, const int32_t* expert_map, const moe_weights* w1,
                      const moe_weights* w2, const LayerOpts& o, const RoutedWs& b,
                      int32_t* map_out, void* y_out, uint16_t* w_bf16_out, hipStream_t s) {
  int32_t* map = map_out ? map_out : b.map;
  void* y = y_out ? y_out : b.x_perm;
  // Rows in the standard layout: GEMM1 reads each permuted row straight from
  // the token rows through the inverse map (no gather kernel, no x_perm write
  // and re-read), while they fit one buffer descriptor's 4 GiB: bf16 rows
  // unless the routing weight goes on them (the gather applies it); two-term
  // FP8 rows with their token's scale (the weight, top-1, was applied before
  // quantizing); one-term FP8 rows only for small batches, where the saved
  // launch counts (measured on prefill batches, their GEMM1 runs 6-11 %
  // slower on gathered rows than on the permuted copy, more than the gather
  // kernel costs); blockwise FP8 keeps the gather (its group scales are read
  // per k-block by rows of the permuted order).
  const int64_t token_row_bytes = o.fp8 ? int64_t(H) * o.terms : int64_t(H) * 2;
  const bool gather_in_gemm =
      (o.fp8 ? !o.block && (o.terms == 2 || T <= kGatherFp8MaxT) : !o.weight_on_input) &&
      o.batch_m == 0 && T * token_row_bytes <= int64_t(0xFFFFFFFF);
  // A small bf16 batch whose GEMM1 takes the decode kernel: router, permute
  // map and GEMM1 in one launch, then GEMM2
  if (!o.fp8 && gather_in_gemm && o.batch_m == 0) {
    const int64_t max_rows = std::min(moe_permuted_rows(T, k), b.rows);
    moe::GemmArgs g1{x, w1->data, scales_of(w1), b.offsets, E_l, H, I, 1, b.rows, b.h, b.split,
                     b.split_bytes, o.act, o.clamp, 0};
    g1.a_inv = b.inv;
    g1.a_k = k;
    g1.a_T = T;
    if (moe::gemm_picks_decode(g1, max_rows) && moe::decode_route_gemm1_fits(g1, T, E, k)) {
      hipError_t e = moe::launch_decode_route_gemm1(logits, T, E, k, score_fn, renormalize, rsf,
                                                    b.ids, b.wts, w_bf16_out, expert_map, map,
                                                    b.offsets, b.inv, b.rows, g1, s);
      if (e != hipSuccess) return hip_fail(e, "route, permute and gemm1");
      moe::GemmArgs g2{b.h, w2->data, scales_of(w2), b.offsets, E_l, I, H, 0, b.rows, y, b.split,
                       b.split_bytes, moe::kActSilu, 0.0f, 0};
      e = moe::launch_grouped_gemm(g2, max_rows, s);
      return e == hipSuccess ? MOE_OK : hip_fail(e, "gemm2");
    }
  }
  // Router and permute map (one launch for a small batch)
  hipError_t e = moe::launch_route_permute(logits, T, E, k, score_fn, renormalize, rsf, b.ids,
                                           b.wts, w_bf16_out, expert_map, E_l, map, b.offsets,
                                           gather_in_gemm ? b.inv : nullptr, b.rows, o.batch_m, s);
  if (e != hipSuccess) return hip_fail(e, "route and permute");
  if (o.weight_on_input && w_bf16_out) {
    e = moe::launch_fill_u16(w_bf16_out, T * k, 0x3F80, s);  // bf16 1.0
    if (e != hipSuccess) return hip_fail(e, "unit weights");
  }
  if (o.block) {
    // Quantize-Dispatch, blockwise: the tokens per 128-element group
    e = moe::launch_quantize_fp8_groups(x, T, H, nullptr, b.xq, b.xs, T, s);
    if (e != hipSuccess) return hip_fail(e, "quantize");
  } else if (o.fp8) {
    // Quantize-Dispatch: the tokens (times their weight when it goes on the
    // input; top_k 1, so one weight per token) to FP8, then their rows
    e = moe::launch_quantize_fp8(x, T, H, o.a1_scale, o.weight_on_input ? b.wts : nullptr,
                                 nullptr, b.xq, b.xs, s, o.terms);
    if (e != hipSuccess) return hip_fail(e, "quantize");
  }
  // (batched experts format: the quantized hidden rows are all E_l * capacity
  // rows, those past an expert's count never read; the standard layout
  // quantizes the offsets[E_l] local routes)
  const int32_t* h_rows = o.batch_m > 0 ? nullptr : b.offsets + E_l;
  if (o.block) {
    e = moe::launch_gather_fp8_rows(b.xq, b.xs, map, T, k, H, b.x_perm, b.ps, s, H / 128, b.rows);
    if (e != hipSuccess) return hip_fail(e, "gather");
    const int64_t max_rows = std::min(moe_permuted_rows(T, k), b.rows);
    moe::GemmArgs g1{b.x_perm, w1->data, scales_of(w1), b.offsets, E_l, H, I, 1, b.rows, b.h,
                     b.split, b.split_bytes, o.act, o.clamp, o.batch_m, b.ps};
    g1.a_ld = b.rows;
    e = moe::launch_grouped_gemm(g1, max_rows, s);
    if (e != hipSuccess) return hip_fail(e, "gemm1");
    // the hidden rows of the local routes, per 128-element group
    e = moe::launch_quantize_fp8_groups(b.h, b.rows, I, h_rows, b.hq, b.hs, b.rows, s);
    if (e != hipSuccess) return hip_fail(e, "quantize hidden");
    moe::GemmArgs g2{b.hq, w2->data, scales_of(w2), b.offsets, E_l, I, H, 0, b.rows, y, b.split,
                     b.split_bytes, moe::kActSilu, 0.0f, o.batch_m, b.hs};
    g2.a_ld = b.rows;
    e = moe::launch_grouped_gemm(g2, max_rows, s);
    if (e != hipSuccess) return hip_fail(e, "gemm2");
    return MOE_OK;
  }
  if (o.fp8) {
    if (!gather_in_gemm) {
      e = moe::launch_gather_fp8_rows(b.xq, b.xs, map, T, k, H * o.terms, b.x_perm, b.ps, s);
      if (e != hipSuccess) return hip_fail(e, "gather");
    }
    const int64_t max_rows = std::min(moe_permuted_rows(T, k), b.rows);
    moe::GemmArgs g1{gather_in_gemm ? static_cast<const void*>(b.xq) : b.x_perm, w1->data,
                     scales_of(w1), b.offsets, E_l, H, I, 1, b.rows, b.h, b.split,
                     b.split_bytes, o.act, o.clamp, o.batch_m, gather_in_gemm ? b.xs : b.ps,
                     w1->dtype == MOE_DTYPE_MXFP4, o.terms};
    if (gather_in_gemm) {
      g1.a_inv = b.inv;
      g1.a_k = k;
      g1.a_T = T;
    }
    e = moe::launch_grouped_gemm(g1, max_rows, s);
    if (e != hipSuccess) return hip_fail(e, "gemm1");
    // the hidden rows of the local routes (offsets[E_l] of them) to FP8
    e = moe::launch_quantize_fp8(b.h, b.rows, I, o.a2_scale, nullptr, h_rows, b.hq, b.hs, s,
                                 o.terms);
    if (e != hipSuccess) return hip_fail(e, "quantize hidden");
    moe::GemmArgs g2{b.hq, w2->data, scales_of(w2), b.offsets, E_l, I, H, 0, b.rows, y, b.split,
                     b.split_bytes, moe::kActSilu, 0.0f, o.batch_m, b.hs,
                     w2->dtype == MOE_DTYPE_MXFP4,
                     o.terms};
    e = moe::launch_grouped_gemm(g2, max_rows, s);
    if (e != hipSuccess) return hip_fail(e, "gemm2");
    return MOE_OK;
  }
  if (!gather_in_gemm) {
    e = moe::launch_gather_rows(x, map, T, k, H, o.weight_on_input ? b.wts : nullptr, b.x_perm,
                                s);
    if (e != hipSuccess) return hip_fail(e, "gather");
  }
  // the tile shape follows the routed rows, the same bound in both formats
  const int64_t max_rows = std::min(moe_permuted_rows(T, k), b.rows);
  moe::GemmArgs g1{gather_in_gemm ? x : b.x_perm, w1->data, scales_of(w1), b.offsets, E_l, H, I,
                   1, b.rows, b.h, b.split, b.split_bytes, o.act, o.clamp, o.batch_m};
  if (gather_in_gemm) {
    g1.a_inv = b.inv;
    g1.a_k = k;
    g1.a_T = T;
  }
  e = moe::launch_grouped_gemm(g1, max_rows, s);
  if (e != hipSuccess) return hip_fail(e, "gemm1");
  moe::GemmArgs g2{b.h, w2->data, scales_of(w2), b.offsets, E_l, I, H, 0, b.rows, y, b.split,
                   b.split_bytes, moe::kActSilu, 0.0f, o.batch_m};
  e = moe::launch_grouped_gemm(g2, max_rows, s);
  if (e != hipSuccess) return hip_fail(e, "gemm2");
  return MOE_OK;
}

static int check_fused_args(const float* logits, const void* x, int64_t T, int32_t H, int32_t I,
                            int32_t E, int32_t E_l, int32_t k, int32_t score_fn,
                            const int32_t* expert_map, const moe_weights* w1,
                            const moe_weights* w2, int64_t pass_T, const LayerOpts& o) {
  MOE_CHECK(check_route_sizes(T, E, k));
  MOE_CHECK(check_local(E, E_l));
  MOE_CHECK(check_gemm_dims(H, I));
  if (score_fn != MOE_SCORE_SOFTMAX && score_fn != MOE_SCORE_SIGMOID)
    return fail(MOE_ERR_UNSUPPORTED, "unknown score function %d", score_fn);
  if (!expert_map && E_l != E)
    return fail(MOE_ERR_INVALID_ARGUMENT, "without an expert map every expert is local (E_l=%d, E=%d)", E_l, E);
  MOE_CHECK(check_weights(w1, "w1"));
  MOE_CHECK(check_weights(w2, "w2"));
  MOE_CHECK(check_pairing(w1, o.fp8, "w1", o.block));
  MOE_CHECK(check_pairing(w2, o.fp8, "w2", o.block));
  if (o.terms == 2 && (w1->dtype != MOE_DTYPE_MXFP4 || w2->dtype != MOE_DTYPE_MXFP4))
    return fail(MOE_ERR_INVALID_ARGUMENT, "two-term FP8 activations need MXFP4 weights");
  if (o.fp8) MOE_CHECK(check_fp8_dims(H, I, w1));
  if (o.batch_m > 0) MOE_CHECK(check_capacity(E_l, o.batch_m));
  const int64_t rows = routed_rows(pass_T, k, E_l, o.batch_m);
  MOE_CHECK(check_gemm_extent(rows, H, 2 * int64_t(I)));
  MOE_CHECK(check_gemm_extent(rows, I, H));
  MOE_CHECK(opt_ptr(expert_map, "expert_map"));
  if (T > 0) {
    MOE_CHECK(need_ptr(logits, "logits"));
    MOE_CHECK(need_ptr(x, "x"));
  }
  return MOE_OK;
}

static int check_workspace(void* workspace, size_t have, size_t need) {
  MOE_CHECK(need_ptr(workspace, "workspace"));
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(MOE_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (have < need) return fail(MOE_ERR_SIZE_MISMATCH, "workspace too small (%zu < %zu bytes)", have, need);
  return MOE_OK;
}

// The deferred form on a given scratch: split_cap bounds the GEMMs' split
// scratch (the rest of the workspace is needed in full).
static int unfinalized_on(const float* logits, const void* x, int64_t T, int32_t H, int32_t I,
                          int32_t E, int32_t E_l, int32_t k, int32_t score_fn,
                          int32_t renormalize, float rsf, const int32_t* expert_map,
                          const moe_weights* w1, const moe_weights* w2, const LayerOpts& o,
                          int64_t R_pad, void* gemm2_permuted, void* expert_weights,
                          int32_t* map, void* workspace, size_t need, size_t split_cap,
                          hipStream_t stream) {
  // the workspace is apart from the input rows and from the three outputs
  if (overlap(workspace, need, x, sizeof(uint16_t) * T * H) ||
      overlap(workspace, need, gemm2_permuted, sizeof(uint16_t) * R_pad * H) ||
      overlap(workspace, need, expert_weights, sizeof(uint16_t) * T * k) ||
      overlap(workspace, need, map, sizeof(int32_t) * T * k))
    return fail(MOE_ERR_DESTINATION_CONFLICT,
                "the workspace must not overlap x, gemm2_permuted, expert_weights or map");
  if (overlap(gemm2_permuted, sizeof(uint16_t) * R_pad * H, x, sizeof(uint16_t) * T * H))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "gemm2_permuted must not overlap x");
  Carve c{static_cast<char*>(workspace)};
  const RoutedWs b = carve_routed(c, T, k, E_l, H, I, o.batch_m, o.fp8, o.terms, split_cap, o.block);
  return run_routed(logits, x, T, H, I, E, E_l, k, score_fn, renormalize, rsf, expert_map, w1, w2,
                    o, b, map, gemm2_permuted, static_cast<uint16_t*>(expert_weights), stream);
}

// Argument checks of the deferred form (everything but the workspace).
static int check_unfinalized(const float* logits, const void* x, int64_t T, int32_t H, int32_t I,
                             int32_t E, int32_t E_l, int32_t k, int32_t score_fn,
                             const int32_t* expert_map, const moe_weights* w1,
                             const moe_weights* w2, const moe_layer_options* options,
                             int64_t R_pad, void* gemm2_permuted, void* expert_weights,
                             int32_t* map, LayerOpts* o) {
  MOE_CHECK(parse_options(options, k, o));
  if (o->chunk > 0 && o->chunk < T)
    return fail(MOE_ERR_INVALID_ARGUMENT, "the deferred form takes no chunking (chunk_tokens < T)");
  MOE_CHECK(check_fused_args(logits, x, T, H, I, E, E_l, k, score_fn, expert_map, w1, w2, T, *o));
  if (o->batch_m > 0) {
    if (R_pad < int64_t(E_l) * o->batch_m)
      return fail(MOE_ERR_SIZE_MISMATCH, "R_pad must hold E_l * batched_max_tokens rows");
  } else {
    MOE_CHECK(check_rpad(T, k, R_pad));
  }
  if (T == 0) return MOE_OK;
  MOE_CHECK(need_ptr(gemm2_permuted, "gemm2_permuted"));
  MOE_CHECK(need_ptr(expert_weights, "expert_weights"));
  return need_ptr(map, "map");
}

int moe_fused_experts_unfinalized(const float* logits, const void* x, int64_t T, int32_t H,
                                  int32_t I, int32_t E, int32_t E_l, int32_t k, int32_t score_fn,
                                  int32_t renormalize, float rsf, const int32_t* expert_map,
                                  const moe_weights* w1, const moe_weights* w2,
                                  const moe_layer_options* options, int64_t R_pad,
                                  void* gemm2_permuted, void* expert_weights, int32_t* map,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  LayerOpts o;
  MOE_CHECK(check_unfinalized(logits, x, T, H, I, E, E_l, k, score_fn, expert_map, w1, w2, options,
                              R_pad, gemm2_permuted, expert_weights, map, &o));
  if (T == 0) return MOE_OK;
  const size_t need = routed_ws_bytes(T, k, E_l, H, I, o.batch_m, o.fp8, o.terms, o.block);
  MOE_CHECK(check_workspace(workspace, workspace_bytes, need));
  return unfinalized_on(logits, x, T, H, I, E, E_l, k, score_fn, renormalize, rsf, expert_map, w1,
                        w2, o, R_pad, gemm2_permuted, expert_weights, map, workspace, need,
                        ~size_t(0), static_cast<hipStream_t>(stream));
}

int moe_fused_experts_unfinalized_noalloc(const float* logits, const void* x, int64_t T,
                                          int32_t H, int32_t I, int32_t E, int32_t E_l, int32_t k,
                                          int32_t score_fn, int32_t renormalize, float rsf,
                                          const int32_t* expert_map, const moe_weights* w1,
                                          const moe_weights* w2, const moe_layer_options* options,
                                          int64_t R_pad, void* gemm2_permuted,
                                          void* expert_weights, int32_t* map, void* stream) {
  g_err[0] = 0;
  LayerOpts o;
  MOE_CHECK(check_unfinalized(logits, x, T, H, I, E, E_l, k, score_fn, expert_map, w1, w2, options,
                              R_pad, gemm2_permuted, expert_weights, map, &o));
  if (T == 0) return MOE_OK;
  // everything but the GEMMs' split scratch must fit; the split scratch takes
  // what is left (fewer split pieces, or none, when little is)
  const int64_t rows = routed_rows(T, k, E_l, o.batch_m);
  const size_t full = routed_ws_bytes(T, k, E_l, H, I, o.batch_m, o.fp8, o.terms, o.block);
  const size_t base = full - align_up(routed_split_bytes(rows, H, I));
  if (base > kNoallocScratchBytes)
    return fail(MOE_ERR_SIZE_MISMATCH,
                "problem needs %zu bytes of scratch, more than the %zu-byte static scratch",
                base, size_t(kNoallocScratchBytes));
  const size_t split_cap = (kNoallocScratchBytes - base) / kAlign * kAlign;
  void* ws = nullptr;
  MOE_CHECK(noalloc_scratch(&ws));
  return unfinalized_on(logits, x, T, H, I, E, E_l, k, score_fn, renormalize, rsf, expert_map, w1,
                        w2, o, R_pad, gemm2_permuted, expert_weights, map, ws,
                        kNoallocScratchBytes, split_cap, static_cast<hipStream_t>(stream));
}

int moe_fused_experts(const float* logits, const void* x, int64_t T, int32_t H, int32_t I,
                      int32_t E, int32_t E_l, int32_t k, int32_t score_fn, int32_t renormalize,
                      float rsf, const int32_t* expert_map, const moe_weights* w1,
                      const moe_weights* w2, int32_t shared_I, const void* ws1, const void* ws2,
                      float rsf_fin, const moe_layer_options* options, void* out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  LayerOpts o;
  MOE_CHECK(parse_options(options, k, &o));
  const int64_t P = pass_tokens(T, o);  // tokens per pass
  MOE_CHECK(check_fused_args(logits, x, T, H, I, E, E_l, k, score_fn, expert_map, w1, w2, P, o));
  if (shared_I < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "shared_I must be >= 0");
  if (shared_I > 0) {
    MOE_CHECK(check_gemm_dims(H, shared_I));
    MOE_CHECK(check_gemm_extent(P, H, 2 * int64_t(shared_I)));
    MOE_CHECK(check_gemm_extent(P, shared_I, H));
  }
  if (T == 0) return MOE_OK;
  MOE_CHECK(need_ptr(out, "out"));
  if (shared_I > 0) {
    MOE_CHECK(need_ptr(ws1, "ws1"));
    MOE_CHECK(need_ptr(ws2, "ws2"));
  }
  size_t shared_bytes = 0;
  MOE_CHECK(moe_shared_workspace_size(P, H, shared_I, &shared_bytes));
  const size_t need = routed_ws_bytes(P, k, E_l, H, I, o.batch_m, o.fp8, o.terms, o.block) + shared_bytes;
  MOE_CHECK(check_workspace(workspace, workspace_bytes, need));
  // out is x itself (in place) or apart from it; the workspace is apart from both
  const size_t row_bytes = sizeof(uint16_t) * T * H;
  if (out != x && overlap(out, row_bytes, x, row_bytes))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "out must be x itself or not overlap it");
  if (overlap(workspace, need, out, row_bytes) || overlap(workspace, need, x, row_bytes))
    return fail(MOE_ERR_DESTINATION_CONFLICT, "the workspace must not overlap x or out");
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carve c{static_cast<char*>(workspace)};
  const RoutedWs b = carve_routed(c, P, k, E_l, H, I, o.batch_m, o.fp8, o.terms, ~size_t(0), o.block);
  int32_t* s_off = nullptr;
  uint16_t* s_h = nullptr;
  uint16_t* s_y = nullptr;
  if (shared_I > 0) {
    s_off = c.take<int32_t>(2);
    s_h = c.take<uint16_t>(P * shared_I);
    s_y = c.take<uint16_t>(P * H);
  }
  // Each pass reads only its own rows of x and writes only its own rows of
  // out, after its last read of them, so out may be x.
  for (int64_t t0 = 0; t0 < T; t0 += P) {
    const int64_t n = std::min(P, T - t0);
    const uint16_t* xc = static_cast<const uint16_t*>(x) + t0 * H;
    MOE_CHECK(run_routed(logits + t0 * E, xc, n, H, I, E, E_l, k, score_fn, renormalize, rsf,
                         expert_map, w1, w2, o, b, nullptr, nullptr, nullptr, s));
    const uint16_t* shared_out = nullptr;
    if (shared_I > 0) {
      // the shared expert is one dense gated MLP: a single-expert grouped
      // GEMM pair over the pass's rows of x
      hipError_t e = moe::launch_fill_i32(s_off, 2, 0, static_cast<int32_t>(n), s);
      if (e != hipSuccess) return hip_fail(e, "shared offsets");
      moe::GemmArgs g1{xc, ws1, nullptr, s_off, 1, H, shared_I, 1, n, s_h, nullptr, 0, o.act,
                       o.clamp};
      e = moe::launch_grouped_gemm(g1, n, s);
      if (e != hipSuccess) return hip_fail(e, "shared gemm1");
      moe::GemmArgs g2{s_h, ws2, nullptr, s_off, 1, shared_I, H, 0, n, s_y};
      e = moe::launch_grouped_gemm(g2, n, s);
      if (e != hipSuccess) return hip_fail(e, "shared gemm2");
      shared_out = s_y;
    }
    hipError_t e = moe::launch_finalize(b.x_perm, b.rows, o.weight_on_input ? nullptr : b.wts, 0, b.map,
                                        n, k, H, rsf_fin, shared_out,
                                        static_cast<uint16_t*>(out) + t0 * H, s);
    if (e != hipSuccess) return hip_fail(e, "finalize");
  }
  return MOE_OK;
}

}  // extern "C"

namespace moe {

int device_cu_count() {
  static int counts[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (counts[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    counts[dev] = n;
  }
  return counts[dev];
}

}  // namespace moe
