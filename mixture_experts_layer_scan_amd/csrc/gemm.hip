// Grouped expert GEMMs (apply() of vLLM's modular fused-MoE kernel: GEMM1,
// the silu-and-mul or gelu-and-mul activation, GEMM2, all unweighted).
//
//   C[r, n] = sum_k A[r, k] * W[e, n, k]     for r in expert e's row segment
//
// Both operands are contiguous along k, which is the natural operand layout
// of the CDNA4 MFMA v_mfma_f32_32x32x16_bf16 (each lane supplies 8 k of one
// row of A and of one row of W), so no transposes are needed.
//
// Work decomposition
//   - Each expert's row segment [offsets[e], offsets[e+1]) is cut into m-tiles
//     of BM rows; tiles of all experts are numbered consecutively.  Every
//     workgroup rebuilds that numbering from `offsets` in LDS (one block scan),
//     so no host synchronisation and no scheduling buffer are needed.
//   - Persistent grid: workgroup b walks tiles slot(b), slot(b) + G, ...  The
//     slot is chosen so that the G/8 workgroups the hardware puts on one XCD
//     (round-robin dispatch) take consecutive tiles, and tiles are ordered in
//     groups of GM m-tiles per n-tile column, so the tiles one XCD runs
//     together share A rows and weight rows in that XCD's L2.  Tiles made for
//     segments of at most BM rows (one m-tile per expert, nothing to share in
//     the weights) use GM = 1: all n-tiles of an expert run on one XCD and
//     read its A rows from HBM once.
//   - Such tiles (one wave row, several 32-row fragments per wave) skip the
//     operand reads and MFMAs of fragments that lie wholly past the segment.
//   - Loads go through buffer descriptors bounded to the expert's row segment
//     and to the expert's weights: rows of a ragged m-tile past the segment
//     read as zero (never another expert's rows) and are masked on store.
//
// Tile pipeline (k-steps of 64; STAGES activation stages, B_STAGES weight
// stages of 128 bytes per weight row: one k-step of bf16, four of e2m1)
//   - Operands move global -> LDS with buffer_load ... lds (16 bytes a lane,
//     straight into LDS, no registers): one wave instruction fills 1 KiB of a
//     stage, 8 rows x 128 bytes.  Rows are stored XOR-swizzled in 16-byte
//     chunks (swz below), the lane choosing the global chunk the swizzle puts
//     at its LDS position, so MFMA operand reads are free of bank conflicts.
//   - k-step kt computes from activation stage kt % STAGES while the loads of
//     k-step kt + STAGES - 1 stream into the stage computed one k-step
//     earlier; a weight stage streams in while the one before it is used.
//   - A k-step ends by waiting until this wave's loads that the next k-step
//     reads have landed (a partial vmcnt: later loads stay in flight; the
//     count comes from a compile-time model of the issue order) and a
//     barrier.  The barrier sits before the last sub-step's MFMAs, and the
//     first operands of the next k-step are read right after it, so LDS read
//     latency hides behind those MFMAs.
//   - Inside a k-step, fenced so the compiler keeps the order: the operand
//     reads of sub-step ks + 1 and a slice of the loads are issued before the
//     MFMAs of sub-step ks.
//
// MXFP4 weights (e2m1 pairs, low nibble = even k, one E8M0 scale byte per 32
// k; vLLM flashinfer_moe_ep.py, _E2M1_LUT and _dequant_fp4_ue8m0_gran32): a
// weight stage holds 256 k of every row (128 packed bytes, so loads fetch
// whole 128-byte row segments, as for bf16).  Each lane reads its 16 packed
// bytes of a k-step once and expands 4 of them per sub-step to bf16 with
// v_cvt_scalef32_pk_bf16_fp4 (value x 2^(s-127), exact in bf16), so the MFMAs
// and the activations stay bf16.  Inside a k-step, sub-step ks and lane half h
// cover k = 32h + 8ks .. +7 for A and W alike, which makes a lane's packed
// bytes of one k-step contiguous and puts all its k in one 32-wide scale
// block.  The scale bytes a lane needs for a weight stage (4 per fragment)
// are loaded into registers one weight stage ahead, right before that
// stage's weight loads: vmcnt retires in issue order, so a wait for them
// never waits for younger weight stages.
//
// Split reduction (tiles for short segments, i.e. decode batches): when the
// tiles are too few to fill the grid, each tile's k-range is cut into S
// pieces on weight-stage boundaries and every (tile, piece) is a work unit.
// S is chosen on the device from the real tile count (a cost model: rounds
// of the persistent grid times the k-steps of a unit plus a fixed fill and
// drain cost), up to the number of fp32 partial slices the workspace holds.
// Pieces write their fp32 sums to slice s of the workspace and
// split_reduce_kernel adds the S slices in order (deterministic, no atomics)
// and applies the activation.
//
// Two-term FP8 activations with MXFP4 weights (bf16 activations split as
// scale * (q1 + q2 / 16), both E4M3): an activation row holds, per 64 k, the
// 64 codes of q1 and then the 64 of q2, so a 128-byte activation stage row is
// one k-step of 64.  Sub-step t multiplies term t by the weight block pair of
// that k-step with the scaled MFMA (A scale 1 or 2^-4, B scale the E8M0 byte),
// both into the same accumulators; the row scale applies in the epilogue.
//
// GEMM1 ("gated"): a tile of BN virtual weight rows holds BN/2 gate rows
// [n0, n0 + BN/2) and the matching BN/2 up rows [I + n0, ...).  Each wave
// computes gate and up blocks with the same lane layout, so the epilogue
// forms act(g) * u in registers and writes BN/2 columns of h.
#include "moe_common.h"

#include <algorithm>
#include <type_traits>
#include <utility>

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int V>
using ic = std::integral_constant<int, V>;

// Calls f(ic<0>), ..., f(ic<N-1>) in order: loop bodies with compile-time
// indices (stage objects, wait counts).
template <class F, int... J>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, J...>) {
  (f(ic<J>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

// Descriptor word 3 for raw (untyped, stride 0) buffer access on gfx9-family
// parts: 32-bit data format, out-of-range offsets read as zero.
constexpr int kBufferFlags = 0x00020000;

// two-term fp8 activations: the second term holds the first one's residual
// times 2^kTerm2Shift
constexpr int kTerm2Shift = 4;

// split-reduction workspace: header (the chosen piece count), then slices
constexpr int64_t kSplitHeader = 256;
constexpr int64_t kMaxSplit = 16;

// tail split (tiles of the whole k-range): a header (tail tile count, pieces
// per tail tile, then row0 / rows / n0 of each tail tile), then one fp32
// [BM, BN] slab per (tail tile, piece)
constexpr int kMaxTail = 64;
constexpr int64_t kTailHeader = 1024;  // >= (2 + 3 * kMaxTail) ints, 256-byte aligned
constexpr int64_t kTailSlabs = 256;    // slabs of the largest tile the scratch holds
constexpr int64_t kTailBytes = kTailHeader + kTailSlabs * 128 * 256 * 4;

// Swizzle of the eight 16-byte chunks of a 128-byte tile row: chunk c of row
// r sits at position c ^ (r & 7) ^ ((r >> 3) & 1), so 16 consecutive rows
// read at one logical chunk (a 16-lane group of an MFMA operand read) hit 16
// distinct 16-byte bank groups of the 64-bank LDS.
__device__ __forceinline__ int swz_key(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// uint16 offset of chunk `chunk` of tile row `row` (rows of 64 uint16).
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 64 + ((chunk ^ swz_key(row)) << 3);
}

// Device-only instructions sit in helpers whose bodies exist only in the
// device pass: the host pass would reject them and silently drop the kernel
// instantiations that use them.

// 16 bytes per lane from buffer `r` at byte offset voff + soff, written
// straight into LDS at dst + 16 * lane (dst is uniform over the wave).
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint16_t* dst, uint32_t voff,
                                          int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, static_cast<int>(voff), soff, 0,
                                           0);
#endif
}

// 4 bytes per lane, written into LDS at dst + 4 * lane.
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t r, float* dst, uint32_t voff,
                                         int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, static_cast<int>(voff), soff, 0,
                                           0);
#endif
}

// Wait until at most N vector-memory loads of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, the other counters
// left open).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
#endif
}

// The same, and every LDS read of this wave has returned (lgkmcnt 0).
template <int N>
__device__ __forceinline__ void wait_vmem_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
#endif
}

// Workgroup barrier without the release/acquire fences of __syncthreads():
// those would wait for every outstanding load of the wave (vmcnt(0)),
// including the direct-to-LDS loads of later k-steps.  Each wave instead
// waits for its own loads of the next stage with wait_vmem before arriving;
// the empty asm statements keep the compiler from moving LDS accesses across.
__device__ __forceinline__ void stage_barrier() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#endif
}

// The value unchanged, but opaque to the optimizer (nothing derived from it
// is hoisted out of the enclosing loop).
__device__ __forceinline__ int opaque(int v) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(v));
#endif
  return v;
}

template <int BM_, int BN_, int WM_, int WN_, int STAGES_, bool GATED_, bool WQ_ = false,
          int GM_ = 8, bool F8_ = false, bool A2_ = false, bool BS_ = false>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = STAGES_;
  static constexpr bool F8 = F8_;  // activations and weights in FP8 E4M3
  // two-term FP8 activations (with MXFP4 weights): 64 codes of the first
  // term, then the 64 of the second term for the same k, per 128 row bytes
  static constexpr bool A2 = A2_;
  static_assert(!A2 || (F8 && WQ_), "two-term activations pair with MXFP4 weights");
  // blockwise FP8: one activation scale per row and 128 k, one weight scale
  // per 128 x 128 block; a k-step (128 k of FP8) is exactly one k-block
  static constexpr bool BS = BS_;
  static_assert(!BS || (F8_ && !WQ_ && !A2_), "block scales pair FP8 activations and weights");
  // k per k-step: 128 bytes of an activation row (64 bf16, 128 fp8, or 64
  // of each of the two fp8 terms)
  static constexpr int BK = A2 ? 64 : F8 ? 128 : 64;
  static constexpr bool GATED = GATED_;
  static constexpr bool WQ = WQ_;  // weights in MXFP4
  static constexpr int GM = GM_;   // m-tiles per group of the tile order
  static constexpr int NWAVES = WM * WN;
  static constexpr int kThreads = NWAVES * kWave;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  // skip row fragments past the segment: in tiles of one wave row, and in
  // the eight-wave weight-streaming tile (2 x 4 waves: each SIMD holds one
  // wave of each wave row, so the skipped work leaves no SIMD idle while
  // another computes); a wave of the lower row may then have no fragment
  static constexpr bool SKIP = (WM == 1 && FM > 1) || (GM == 1 && WM > 1);
  // one wave row: the tiles for short segments, which may split the k-range
  static constexpr bool SPLIT = (WM == 1);
  // MFMA sub-steps per k-step: 32x32x16 bf16, or 32x32x64 fp8 (two-term:
  // one per term, both with the same weight fragment)
  static constexpr int SUBSTEPS = A2 ? 2 : F8 ? BK / 64 : BK / 16;
  // two stages: the next k-step's loads all go out with the first sub-step,
  // since they must land by the end of this one
  static constexpr bool EARLY = (STAGES == 2);
  static constexpr int OUT_N = GATED ? BN / 2 : BN;
  // one load instruction: 8 rows x 128 bytes
  static constexpr int A_LD = BM / 8 / NWAVES;   // activation loads per wave per k-step
  static constexpr int B_LD = BN / 8 / NWAVES;   // weight loads per wave per weight stage
  // k-steps per weight stage (128 bytes of a weight row: 256 k of e2m1)
  static constexpr int B_KS = WQ ? (F8 && !A2 ? 2 : 4) : 1;
  // MXFP4: three weight stages, so two stream while one is used (a weight
  // stage lasts four k-steps; with one in flight the stream stalls between)
  static constexpr int B_STAGES = WQ ? 3 : STAGES;
  // scale loads per wave per weight stage: one 8-byte load per fragment (rows
  // of K/32 scale bytes 8-byte aligned); the byte-wise fallback for other K
  // issues more, which only makes the waits stricter
  static constexpr int SCQ = WQ ? FN : 0;
  // blockwise FP8: the activation scales of a k-step's rows travel with its
  // activation loads, one 4-byte direct-to-LDS load per wave (its wave row's
  // rows, 64 lanes: wave tiles of at most 64 rows), into a scale stage of
  // SC_N floats per activation stage
  static constexpr int SAQ = BS ? 1 : 0;
  static constexpr int SC_N = BS ? WM * 64 : 4;
  static constexpr int A_ELEMS = BM * 64;        // uint16 per activation stage
  static constexpr int B_ELEMS = BN * 64;        // uint16 per weight stage
  // k-steps per unrolled loop body: every stage object is then compile-time
  static constexpr int UNROLL = STAGES * (B_KS * B_STAGES) / gcd_c(STAGES, B_KS * B_STAGES);

  // ---- model of the load issue order, for the end-of-k-step vmcnt waits ----
  // Prologue: the scale bytes of weight stage 0; then, for bf16, the
  // activation and weight loads of k-steps 0 .. STAGES-2 (stage by stage),
  // for MXFP4 the weight stages 0 .. B_STAGES-2 and then the activation loads
  // of k-steps 0 .. STAGES-2.  k-step kt: when it opens a weight stage q, the
  // scale bytes of stage q + 1; then (spread over its sub-steps) the
  // activation loads of kt + STAGES - 1 and, when it opens a weight stage,
  // the weight loads of the stage B_STAGES - 1 ahead.
  static constexpr int loads_at(int kt) {
    return A_LD + SAQ + (kt % B_KS == 0 ? B_LD + SCQ : 0);
  }
  static constexpr int sum_loads(int from, int to) {
    int n = 0;
    for (int j = from; j <= to; ++j) n += loads_at(j);
    return n;
  }
  // prologue loads issued after the activation loads of k-step s / after the
  // weight loads of stage q (whole groups only: conservative)
  static constexpr int pro_after_a(int s) {
    return B_KS == 1 ? (STAGES - 2 - s) * (A_LD + SAQ + B_LD) : (STAGES - 2 - s) * A_LD;
  }
  static constexpr int pro_after_b(int q) {
    return B_KS == 1 ? (STAGES - 2 - q) * (A_LD + SAQ + B_LD)
                     : (B_STAGES - 2 - q) * B_LD + (STAGES - 1) * A_LD;
  }
  // Loads that may stay in flight at the end of k-step kt with the
  // activation loads of kt + 1 landed, and its weight stage when kt + 1 opens
  // one: only loads issued in later k-steps (or later in the prologue) count.
  static constexpr int need(int kt) {
    const int ia = kt + 2 - STAGES;  // k-step that issued the activations of kt + 1
    int n = ia >= 0 ? sum_loads(ia + 1, kt) : pro_after_a(kt + 1) + sum_loads(0, kt);
    if ((kt + 1) % B_KS == 0) {
      const int q = (kt + 1) / B_KS;
      const int ib = (q - (B_STAGES - 1)) * B_KS;  // k-step that issued weight stage q
      const int nb = ib >= 0 ? sum_loads(ib + 1, kt) : pro_after_b(q) + sum_loads(0, kt);
      n = nb < n ? nb : n;
    }
    return n;
  }
  // the count for every k-step at position j of the unrolled body (minimum
  // over the first bodies, which include the prologue transient)
  static constexpr int wait_at(int j) {
    int n = 63;
    for (int kt = j; kt < 4 * UNROLL + 2 * (STAGES + B_KS * B_STAGES); kt += UNROLL) {
      const int m = need(kt);
      n = m < n ? m : n;
    }
    return n;
  }
  static constexpr int WAIT_PRO = pro_after_a(0) < pro_after_b(0) ? pro_after_a(0) : pro_after_b(0);

  static constexpr bool waits_fit() {
    for (int j = 0; j < UNROLL; ++j)
      if (wait_at(j) < 0 || wait_at(j) >= 64) return false;
    return WAIT_PRO >= 0 && WAIT_PRO < 64;
  }
  static_assert(waits_fit(), "in-flight loads must fit vmcnt");
  static_assert(STAGES >= 2 && STAGES <= 4 && B_STAGES >= 2 && B_STAGES <= 4, "stages");
  static_assert(UNROLL <= 12, "unrolled body");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(!GATED || (FN % 2 == 0), "gated tiles pair gate and up blocks");
  static_assert(!BS || WTM <= 64, "one scale load covers a wave row of at most 64 rows");
  static_assert(BM % (8 * NWAVES) == 0 && BN % (8 * NWAVES) == 0, "whole load instructions");
};

// First virtual weight row of fragment fn of wave column wn.
template <class Cfg>
__device__ __forceinline__ int b_row0(int wn, int fn) {
  constexpr int FN = Cfg::FN;
  if (Cfg::GATED)
    return (fn < FN / 2) ? wn * (Cfg::WTN / 2) + fn * 32
                         : Cfg::BN / 2 + wn * (Cfg::WTN / 2) + (fn - FN / 2) * 32;
  return wn * Cfg::WTN + fn * 32;
}

__device__ __forceinline__ uint32_t load_byte(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, static_cast<int>(voff), soff, 0);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 load_u128(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), soff, 0);
}

__device__ __forceinline__ uint32_t load_u32(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(voff), soff, 0);
}

__device__ __forceinline__ u32x2 load_u64(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(voff), soff, 0);
}

// E8M0 scale byte -> the float whose bit pattern is s << 23 (2^(s-127);
// s = 0 gives 0, s = 255 gives +inf).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) { return __uint_as_float(s << 23); }

// 8 e2m1 values (4 bytes, low nibble first) times `scale` -> 8 bf16.
__device__ __forceinline__ bf16x8 expand_fp4x8(uint32_t w, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::kThreads) void grouped_gemm_kernel(
    const void* __restrict__ A, const void* __restrict__ W,
    const void* __restrict__ W_scales, const int32_t* __restrict__ offsets, int E_l, int K,
    int N_out, int64_t R_pad, uint16_t* __restrict__ C, int n_tiles, float* __restrict__ partials,
    int s_cap, int* __restrict__ split_out, int act, float clamp, int batch_m,
    const float* __restrict__ A_scales, const int32_t* __restrict__ a_inv, int a_k,
    int64_t a_T, char* __restrict__ tail_ws, int slab_cap, int64_t a_ld) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, FM = Cfg::FM, FN = Cfg::FN;
  constexpr int NT = Cfg::kThreads, ST = Cfg::STAGES, SUB = Cfg::SUBSTEPS;
  constexpr int SB = Cfg::B_STAGES, BKS = Cfg::B_KS, U = Cfg::UNROLL;
  using Frag = typename std::conditional<Cfg::F8, i32x8, bf16x8>::type;
  const int kind = act_kind(act, clamp);  // GEMM1 epilogue: 0 silu, 1 clamped silu, 2 gelu
  const float cl = act_limit(clamp);
  // LDS stages as distinct objects, so the compiler knows that loads into one
  // never alias operand reads from another (unused ones are tiny)
  __shared__ __attribute__((aligned(16))) uint16_t lds_a0[Cfg::A_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t lds_a1[Cfg::A_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t lds_a2[ST > 2 ? Cfg::A_ELEMS : 8];
  __shared__ __attribute__((aligned(16))) uint16_t lds_a3[ST > 3 ? Cfg::A_ELEMS : 8];
  __shared__ __attribute__((aligned(16))) uint16_t lds_b0[Cfg::B_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t lds_b1[Cfg::B_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t lds_b2[SB > 2 ? Cfg::B_ELEMS : 8];
  __shared__ __attribute__((aligned(16))) uint16_t lds_b3[SB > 3 ? Cfg::B_ELEMS : 8];
  __shared__ __attribute__((aligned(16))) float lds_c0[Cfg::SC_N];
  __shared__ __attribute__((aligned(16))) float lds_c1[Cfg::SC_N];
  __shared__ __attribute__((aligned(16))) float lds_c2[ST > 2 ? Cfg::SC_N : 4];
  __shared__ __attribute__((aligned(16))) float lds_c3[ST > 3 ? Cfg::SC_N : 4];
  __shared__ int32_t s_mt[1025];
  __shared__ int32_t s_scratch[16];

  // stage objects by compile-time index (taken modulo the stage count)
  auto a_stage = [&](auto i) -> uint16_t* {
    constexpr int s = decltype(i)::value % ST;
    if constexpr (s == 0) return lds_a0;
    else if constexpr (s == 1) return lds_a1;
    else if constexpr (s == 2) return lds_a2;
    else return lds_a3;
  };
  auto b_stage = [&](auto i) -> uint16_t* {
    constexpr int s = decltype(i)::value % SB;
    if constexpr (s == 0) return lds_b0;
    else if constexpr (s == 1) return lds_b1;
    else if constexpr (s == 2) return lds_b2;
    else return lds_b3;
  };
  // blockwise FP8: the activation scale stage beside each activation stage
  auto c_stage = [&](auto i) -> float* {
    constexpr int s = decltype(i)::value % ST;
    if constexpr (s == 0) return lds_c0;
    else if constexpr (s == 1) return lds_c1;
    else if constexpr (s == 2) return lds_c2;
    else return lds_c3;
  };

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;

  // Expert e's rows: [offsets[e], offsets[e+1]), or in the batched experts
  // format [e * batch_m, e * batch_m + min(offsets[e], batch_m)).
  auto seg_start = [&](int e) -> int { return batch_m > 0 ? e * batch_m : offsets[e]; };
  auto seg_rows = [&](int e) -> int {
    return batch_m > 0 ? min(max(offsets[e], 0), batch_m) : offsets[e + 1] - offsets[e];
  };

  // m-tile numbering: s_mt[e] = m-tiles of experts < e.
  {
    const int per = (E_l + NT - 1) / NT;
    int local = 0;
    for (int i = 0; i < per; ++i) {
      const int e = tid * per + i;
      if (e < E_l) local += (seg_rows(e) + BM - 1) / BM;
    }
    int total_m = 0;
    int run = block_exclusive_sum(local, s_scratch, &total_m);
    for (int i = 0; i < per; ++i) {
      const int e = tid * per + i;
      if (e < E_l) {
        s_mt[e] = run;
        run += (seg_rows(e) + BM - 1) / BM;
      }
    }
    if (tid == 0) s_mt[E_l] = total_m;
    __syncthreads();
  }
  const int total_m = s_mt[E_l];
  const int total_tiles = total_m * n_tiles;
  const int G = gridDim.x;
  const int slot = (G % 8 == 0) ? static_cast<int>(blockIdx.x % 8) * (G / 8) + blockIdx.x / 8
                                : static_cast<int>(blockIdx.x);
  const int N_total = Cfg::GATED ? 2 * N_out : N_out;
  const int nk_all = K / BK;                  // k-steps
  const int nq_all = (nk_all + BKS - 1) / BKS;  // weight stages
  // pieces per tile: the S <= s_cap (and at least 4 k-steps a piece) that
  // minimises rounds * (k-steps per piece + fixed cost); 1 without partials
  int S = 1;
  if (Cfg::SPLIT && partials != nullptr && total_tiles > 0) {
    constexpr int kFixed = 8;  // fill, drain and epilogue of a unit, in k-steps
    const int s_max = min(min(s_cap, nq_all), max(1, nk_all / 4));
    long best = -1;
    for (int c = 1; c <= s_max; ++c) {
      const long rounds = (static_cast<long>(total_tiles) * c + G - 1) / G;
      const long cost = rounds * ((nk_all + c - 1) / c + kFixed);
      if (best < 0 || cost < best) { best = cost; S = c; }
    }
  }
  if (split_out != nullptr && blockIdx.x == 0 && tid == 0) split_out[tid] = S;
  // Tail split (tiles of the whole k-range): when the last round of the
  // persistent grid would hold only a few tiles, each of them is cut along
  // k into pieces so that round is full; the pieces write fp32 slabs and
  // tail_reduce_kernel adds them in order.
  int tail_n = 0, St = 1;
  if (!Cfg::SPLIT && tail_ws != nullptr) {
    const int tail = total_tiles % G;
    if (tail > 0 && tail <= kMaxTail && total_tiles > G) {
      const int c = min(min(G / tail, static_cast<int>(kMaxSplit)), nq_all);
      if (c >= 2 && tail * c <= slab_cap) {
        tail_n = tail;
        St = c;
      }
    }
  }
  int* const tail_hdr = reinterpret_cast<int*>(tail_ws);
  if (tail_ws != nullptr && blockIdx.x == 0 && tid == 0) {
    tail_hdr[0] = tail_n;
    tail_hdr[1] = St;
  }
  const int head_tiles = total_tiles - tail_n;
  const int head_units = head_tiles * S;
  const int total_units = head_units + tail_n * St;

  // Load j of this wave fills tile rows [8 rb, 8 rb + 8) (rb = j * NWAVES +
  // wave); lane L writes the 16 bytes at LDS row 8 rb + L / 8, position L % 8,
  // so it fetches the logical chunk the swizzle puts there.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int ld_sub = lane >> 3;
  const int ld_pos = lane & 7;

  for (int unit = slot; unit < total_units; unit += G) {
    const bool in_tail = unit >= head_units;
    const int tile = in_tail ? head_tiles + (unit - head_units) / St : unit / S;
    const int piece = in_tail ? (unit - head_units) % St : unit - tile * S;
    const int S_u = in_tail ? St : S;
    // this piece's weight stages [q0, q0 + nq) and k-steps [kt0, kt0 + nk)
    const int q0 = piece * nq_all / S_u;
    const int nq = (piece + 1) * nq_all / S_u - q0;
    const int kt0 = q0 * BKS;
    const int nk = min(nk_all - kt0, nq * BKS);
    // grouped order: GM m-tiles share each n-tile column
    const int group = Cfg::GM * n_tiles;
    const int gid = tile / group;
    const int first_m = gid * Cfg::GM;
    const int gm = min(total_m - first_m, Cfg::GM);
    const int in_group = tile - gid * group;
    const int m_tile = first_m + in_group % gm;
    const int n_tile = in_group / gm;

    int lo = 0, hi = E_l;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_mt[mid] <= m_tile) lo = mid; else hi = mid;
    }
    // the tile's expert and rows are the same in every lane: held in scalar
    // registers, so the branches on them below are scalar branches
    const int e = __builtin_amdgcn_readfirstlane(lo);
    const int s0 = seg_start(e);
    const int seg_end = min(static_cast<int64_t>(s0) + seg_rows(e), R_pad);
    const int row0 = __builtin_amdgcn_readfirstlane(s0 + (m_tile - s_mt[e]) * BM);
    const int rows = __builtin_amdgcn_readfirstlane(seg_end - row0);
    if (rows <= 0) continue;
    const int n0 = n_tile * Cfg::OUT_N;
    // row fragments of this wave that hold rows of the segment (wave-uniform;
    // at least 1 with one wave row, possibly 0 or less for a lower wave row)
    const int fm_act = __builtin_amdgcn_readfirstlane(
        Cfg::SKIP ? min(FM, (rows - wm * Cfg::WTM + 31) / 32) : FM);

    // Buffer descriptors: A over rows [row0, seg_end) of this expert (or,
    // gathered, over all token rows, rows past the segment given an offset
    // past the end), W over this expert's weights; loads past either range
    // return zero.
    // activation bytes per row: K * 2 (bf16) or K (fp8)
    // (two-term fp8: K * 2, both terms)
    const uint32_t a_row_bytes = (Cfg::F8 && !Cfg::A2) ? static_cast<uint32_t>(K)
                                                       : static_cast<uint32_t>(K) * 2u;
    const bool gathered = a_inv != nullptr;  // uniform
    const uint32_t a_span = gathered ? static_cast<uint32_t>(a_T) * a_row_bytes
                                     : static_cast<uint32_t>(rows) * a_row_bytes;
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(A) +
                             (gathered ? 0 : static_cast<int64_t>(row0) * a_row_bytes)),
        0, static_cast<int>(a_span), kBufferFlags);
    // weight bytes per row: K * 2 (bf16), K / 2 (packed e2m1) or K (fp8)
    const uint32_t w_row_bytes = Cfg::WQ ? static_cast<uint32_t>(K) / 2u
                                 : Cfg::F8 ? static_cast<uint32_t>(K)
                                           : static_cast<uint32_t>(K) * 2u;
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(W) +
                             static_cast<int64_t>(e) * N_total * w_row_bytes),
        0, static_cast<int>(static_cast<uint32_t>(N_total) * w_row_bytes), kBufferFlags);
    // Weight rows a power of two apart put the 128-byte segments that the
    // concurrent tiles of an XCD read at one k-step at the same offset in
    // every row, which bunches them onto few HBM channels.  Such
    // weight-streaming tiles (one m-tile per expert, all n-tiles of an expert
    // at once) start their k-range at a tile-dependent weight stage and wrap
    // around, so concurrent tiles read different offsets (the sum order
    // changes with the tile, and is the same on every run).
    const int rq = (Cfg::GM == 1 && nq > 0 && nk == nq * BKS && (w_row_bytes & (w_row_bytes - 1)) == 0)
                       ? static_cast<int>(tile % nq) : 0;
    auto qrot = [&](int q) {
      const int v = q + rq;
      return v >= nq ? v - nq : v;
    };
    auto krot = [&](int kt) { return qrot(kt / BKS) * BKS + kt % BKS; };
    uint32_t a_off[Cfg::A_LD];
#pragma unroll
    for (int j = 0; j < Cfg::A_LD; ++j) {
      const int r = (j * Cfg::NWAVES + wave_u) * 8 + ld_sub;
      const int c = ld_pos ^ swz_key(r);
      if (gathered) {
        // the token of permuted row row0 + r; past the segment, past the end
        const int32_t x = r < rows ? a_inv[row0 + r] : -1;
        a_off[j] = x >= 0 ? static_cast<uint32_t>(x / a_k) * a_row_bytes + c * 16u : a_span;
      } else {
        a_off[j] = static_cast<uint32_t>(r) * a_row_bytes + c * 16u;
      }
    }
    // gated: virtual rows [0, BN/2) are gate rows n0 + v, the rest up rows
    // I + n0 + v - BN/2; columns past N_out are loaded but never stored
    auto wrow_of = [&](int v) {
      return Cfg::GATED ? (v < BN / 2 ? n0 + v : N_out + n0 + v - BN / 2) : n0 + v;
    };
    uint32_t b_off[Cfg::B_LD];
#pragma unroll
    for (int j = 0; j < Cfg::B_LD; ++j) {
      const int v = (j * Cfg::NWAVES + wave_u) * 8 + ld_sub;
      const int c = ld_pos ^ swz_key(v);
      b_off[j] = static_cast<uint32_t>(wrow_of(v)) * w_row_bytes + c * 16;
    }
    // MXFP4 scale bytes: lane's weight row per fragment; k-step kt, half h
    // uses block 2 kt + h, i.e. byte 2 p + h of the 8 of its weight stage.
    // A lane holds the stage's 8 bytes of its row (both halves' blocks) in
    // two dwords, loaded with one 8-byte load when the rows of K/32 bytes
    // are 8-byte aligned, else byte by byte (its half's 4 bytes) and packed
    // when the stage opens.
    const uint32_t s_row = Cfg::WQ ? static_cast<uint32_t>(K) / 32u : 0u;  // scale bytes per row
    const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(W_scales) +
                             static_cast<int64_t>(e) * N_total * s_row), 0,
        static_cast<int>(static_cast<uint32_t>(N_total) * s_row), kBufferFlags);
    // (FP8 activations with MXFP4 weights need K % 256 == 0: always wide)
    const bool s_wide = Cfg::F8 || (s_row % 8u) == 0;  // uniform
    constexpr int NSF = Cfg::WQ ? FN : 1;
    uint32_t s_off[NSF];
    u32x2 sc_cur[NSF], sc_nxt[NSF];
    uint32_t sc_byte[NSF][4];
    if constexpr (Cfg::WQ) {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        s_off[fn] = static_cast<uint32_t>(wrow_of(b_row0<Cfg>(wn, fn) + (lane & 31))) * s_row;
    }
    // the scale bytes of weight stage q (blocks 8q .. 8q + 7 of the lane's row)
    auto load_scales = [&](int q) {
      if constexpr (Cfg::WQ) {
        if (s_wide) {
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) sc_nxt[fn] = load_u64(s_rsrc, s_off[fn], (q0 + qrot(q)) * 8);
        } else if constexpr (!Cfg::F8) {
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int p = 0; p < 4; ++p)
              sc_byte[fn][p] = load_byte(s_rsrc, s_off[fn] + 2 * p + (lane >> 5), (q0 + qrot(q)) * 8);
        }
      }
    };
    // at a weight-stage boundary (the loads were issued a stage earlier)
    auto rotate_scales = [&]() {
      if constexpr (Cfg::WQ) {
        const uint32_t sh = 8u * static_cast<uint32_t>(lane >> 5);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          if (s_wide || Cfg::F8) {
            sc_cur[fn] = sc_nxt[fn];
          } else {
            sc_cur[fn] = u32x2{(sc_byte[fn][0] << sh) | (sc_byte[fn][1] << (16u + sh)),
                               (sc_byte[fn][2] << sh) | (sc_byte[fn][3] << (16u + sh))};
          }
        }
      }
    };
    // E8M0 scale of fragment fn for the k-step at position p, this lane's half
    auto scale_of = [&](int fn, int p, int ln) {
      const uint32_t word = p < 2 ? sc_cur[fn].x : sc_cur[fn].y;
      return e8m0_to_f32((word >> (8u * static_cast<uint32_t>(2 * (p & 1) + (ln >> 5)))) & 0xFFu);
    };
    // FP8 activations x MXFP4 weights: the E8M0 byte of fragment fn's block
    // 4p + 2ks + h of the weight stage (k-step position p, sub-step ks, half
    // h), handed to the MFMA as its B block scale
    auto scale_byte = [&](int fn, int p, int ks, int ln) -> int {
      const int block = Cfg::A2 ? 2 * p + (ln >> 5) : 4 * p + 2 * ks + (ln >> 5);
      const uint32_t word = block < 4 ? sc_cur[fn].x : sc_cur[fn].y;
      return static_cast<int>((word >> (8u * static_cast<uint32_t>(block & 3))) & 0xFFu);
    };

    // Blockwise FP8: the scales of k-block kb for the tile's rows (A scales
    // stored k-block-major, [K / 128][a_ld]) and for the weight fragments'
    // 128-row blocks ([E_l][N_total / 128][K / 128]), applied after a
    // k-step's MFMAs: acc += sum_k * a_scale[row] * w_scale.  The row scales
    // of a k-step ride with its activation loads into the scale stage beside
    // its activation stage (each wave loads its wave row's 64 rows; reads
    // past the array return zero, and rows past the segment are never
    // stored); at the top of the k-step each lane reads its 16 rows' scales
    // per row fragment from there, before the barrier that frees the stage.
    // The weight scales are wave-uniform: read through the scalar cache.
    constexpr int BSM = Cfg::BS ? FM : 1, BSN = Cfg::BS ? FN : 1;
    u32x4 bs_a[BSM][4];
    uint32_t bs_w[BSN];
    // the uniform index of each weight fragment's scale row (the last block
    // row for virtual weight rows past N_total, whose results are never
    // stored)
    int bs_wblk[BSN];
    const int nkb = K / BK;
    const int nb_rows = N_total / 128;
    const int wm_u = wave_u / Cfg::WN;
    const __amdgpu_buffer_rsrc_t bs_arsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(A_scales), 0,
        Cfg::BS ? static_cast<int>(static_cast<int64_t>(nkb) * a_ld * 4) : 0, kBufferFlags);
    const uint32_t* const bs_wsc =
        static_cast<const uint32_t*>(W_scales) + (Cfg::BS ? static_cast<int64_t>(e) * nb_rows * nkb : 0);
    if constexpr (Cfg::BS) {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        bs_wblk[fn] = __builtin_amdgcn_readfirstlane(
            min(wrow_of(b_row0<Cfg>(wn, fn)) / 128, nb_rows - 1) * nkb);
    }
    // k-block of k-step kt (the k-order may start at a tile-dependent stage)
    auto kblock = [&](int kt) { return kt0 + krot(kt); };
    // this k-step's scales: the rows' from scale stage `cs`, the weights'
    auto load_bscales = [&](int kt, const float* cs) {
      if constexpr (Cfg::BS) {
        const int kb = kblock(kt);
        const int half = lane >> 5;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            bs_a[fm][g] = *reinterpret_cast<const u32x4*>(
                cs + wm * 64 + fm * 32 + 8 * g + 4 * half);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) bs_w[fn] = bs_wsc[bs_wblk[fn] + kb];
      }
    };

    f32x16 acc[FM][FN];
    f32x16 tmp[Cfg::BS ? FM : 1][Cfg::BS ? FN : 1];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    // Slice `part` (of SUB) of the activation loads of k-step kt into stage
    // `st`, and of the weight loads of weight stage q into `wst`: the loads
    // are spread over the sub-steps of the k-step that issues them.
    // (blockwise FP8: with the first slice, the k-step's row scales of this
    // wave's wave row into scale stage `cst`)
    auto gload_a = [&](uint16_t* st, float* cst, int kt, int part) {
#pragma unroll
      for (int j = 0; j < Cfg::A_LD; ++j)
        if (Cfg::EARLY ? part == 0 : j % SUB == part)
          lds_dma16(a_rsrc, st + (j * Cfg::NWAVES + wave_u) * 512, a_off[j], (kt0 + krot(kt)) * 128);
      if constexpr (Cfg::BS)
        if (part == 0)
          lds_dma4(bs_arsrc, cst + wm_u * 64,
                   static_cast<uint32_t>(kblock(kt) * a_ld + row0 + wm_u * Cfg::WTM + lane) * 4u, 0);
    };
    auto gload_b = [&](uint16_t* wst, int q, int part) {
#pragma unroll
      for (int j = 0; j < Cfg::B_LD; ++j)
        if (Cfg::EARLY ? part == 0 : (j + Cfg::A_LD) % SUB == part)
          lds_dma16(b_rsrc, wst + (j * Cfg::NWAVES + wave_u) * 512, b_off[j], (q0 + qrot(q)) * 128);
    };

    // Operand fragments of sub-step ks of the k-step at position p of its
    // weight stage, from activation stage `as` and weight stage `bs`: lane
    // half h holds k = 32h + 8ks .. +7 of its A row and of its W row.  `ln` is
    // the lane id made opaque per k-step so the (swizzled) addresses are
    // rebuilt there instead of all being kept live.  MXFP4: at ks == 0 the
    // lane's 16 packed bytes of the k-step (chunk 2p + h of its row) are read
    // into `bq`; every sub-step expands 4 of them (sub-step 0's at the top of
    // the k-step: see expand0).
    // FP8: lane half h of sub-step ks holds the 32 bytes of chunks 4h + 2ks
    // and 4h + 2ks + 1 of its A row and of its W row (k = 64 ks + 32 h ..
    // + 31 of the k-step); the 32x32x64 MFMA runs unscaled (E8M0 127 = 1),
    // the per-row and per-channel scales apply in the epilogue.
    // FP8 x e2m1: a B lane holds one 32-k block of its weight row (block
    // 4p + 2ks + h of the weight stage: its 16 bytes and its E8M0 scale);
    // the MFMA pairs the first 16 values of A half h with B half 0's values
    // 16h .. 16h + 15 and the last 16 with B half 1's, so A half h reads the
    // 16-byte halves h of blocks 2ks and 2ks + 1: chunks 4ks + h, 4ks + 2 + h.
    auto load_frags = [&](const uint16_t* as, const uint16_t* bs, int ln, int ks, int p,
                          Frag* af, Frag* bfr, uint4* bq) {
      const int frag_row = ln & 31;
      const int half = ln >> 5;
      const int chunk = Cfg::F8 ? half * 4 + 2 * ks : half * SUB + ks;
      // FP8 A chunks (see above)
      const int a_lo = Cfg::WQ ? 4 * ks + half : chunk;
      const int a_hi = Cfg::WQ ? 4 * ks + 2 + half : chunk + 1;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        if (Cfg::SKIP && fm >= fm_act) continue;
        const int r = wm * Cfg::WTM + fm * 32 + frag_row;
        if constexpr (Cfg::F8) {
          const uint4 lo = *reinterpret_cast<const uint4*>(as + swz(r, a_lo));
          const uint4 hi = *reinterpret_cast<const uint4*>(as + swz(r, a_hi));
          af[fm] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                         (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        } else {
          af[fm] = *reinterpret_cast<const bf16x8*>(as + swz(r, chunk));
        }
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int v = b_row0<Cfg>(wn, fn) + frag_row;
        if constexpr (Cfg::F8 && Cfg::WQ) {
          // the 32 e2m1 values (low nibble first) of block 4p + 2ks + h
          // (two-term: block 2p + h in both sub-steps)
          const int blk = Cfg::A2 ? 2 * p + half : 4 * p + 2 * ks + half;
          const uint4 q = *reinterpret_cast<const uint4*>(bs + swz(v, blk));
          bfr[fn] = i32x8{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
        } else if constexpr (Cfg::F8) {
          const uint4 lo = *reinterpret_cast<const uint4*>(bs + swz(v, chunk));
          const uint4 hi = *reinterpret_cast<const uint4*>(bs + swz(v, chunk + 1));
          bfr[fn] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                          (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        } else if constexpr (Cfg::WQ) {
          if (ks == 0) {
            bq[fn] = *reinterpret_cast<const uint4*>(bs + swz(v, 2 * p + half));
          } else {
            const uint32_t word = ks == 1 ? bq[fn].y : ks == 2 ? bq[fn].z : bq[fn].w;
            bfr[fn] = expand_fp4x8(word, scale_of(fn, p, ln));
          }
        } else {
          bfr[fn] = *reinterpret_cast<const bf16x8*>(bs + swz(v, chunk));
        }
      }
    };

    // Operand fragments, double-buffered by sub-step; buffer 0 holds sub-step
    // 0 of the next k-step when a k-step begins.
    static_assert(SUB % 2 == 0, "sub-step 0 of the next k-step reuses buffer 0");
    Frag fa[2][FM], fb[2][FN];
    uint4 bq[Cfg::WQ ? FN : 1];
    // MXFP4: sub-step 0's weight fragments from the packed words read after
    // the previous barrier.  Expanding them there would stall the in-order
    // issue on that LDS read ahead of the last MFMAs; here those MFMAs are
    // already in flight.
    auto expand0 = [&](int p) {
      if constexpr (Cfg::WQ && !Cfg::F8) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          fb[0][fn] = expand_fp4x8(bq[fn].x, scale_of(fn, p, lane));
      }
    };

    // k-step kt at position J of the unrolled body: computes from activation
    // stage J and weight stage J / BKS; streams the activations of k-step
    // kt + ST - 1 into activation stage J - 1 (computed in the previous
    // k-step, which the barrier closed) and, when J opens a weight stage, the
    // weight stage SB - 1 ahead into the one the previous weight stage used;
    // the last k-steps reload the final ones into stages nobody reads again.
    auto kstep = [&](auto jc, int kt) {
      constexpr int J = decltype(jc)::value;
      constexpr int P = J % BKS;  // position inside the weight stage
      uint16_t* const cur_a = a_stage(ic<J>{});
      uint16_t* const nxt_a = a_stage(ic<J + 1>{});
      uint16_t* const ld_a = a_stage(ic<J + ST - 1>{});
      float* const ld_c = c_stage(ic<J + ST - 1>{});
      uint16_t* const cur_b = b_stage(ic<J / BKS>{});
      uint16_t* const nxt_b = b_stage(ic<(J + 1) / BKS>{});
      uint16_t* const ld_b = b_stage(ic<J / BKS + SB - 1>{});
      const int kn = min(kt + ST - 1, nk - 1);
      const int qn = min(kt / BKS + SB - 1, nq - 1);
      if constexpr (P == 0) {
        // scales of this weight stage (loaded a stage ago), then those of the
        // next one, ahead of this k-step's tile loads as the wait model counts
        rotate_scales();
        load_scales(min(kt / BKS + 1, nq - 1));
      }
      // blockwise FP8: this k-step's block scales
      load_bscales(kt, c_stage(ic<J>{}));
      expand0(P);
      const int ln = opaque(lane);
#pragma unroll
      for (int ks = 0; ks < SUB; ++ks) {
        if (ks + 1 < SUB)
          load_frags(cur_a, cur_b, ln, ks + 1, P, fa[(ks + 1) & 1], fb[(ks + 1) & 1], bq);
        gload_a(ld_a, ld_c, kn, ks);
        if constexpr (P == 0) gload_b(ld_b, qn, ks);
        if (ks + 1 == SUB) {
          // this wave's loads that k-step kt + 1 reads landed and its reads
          // of the current stages returned; after the barrier, every wave's
          wait_vmem_lds<Cfg::wait_at(J)>();
          stage_barrier();
          load_frags(nxt_a, nxt_b, ln, 0, (J + 1) % BKS, fa[0], fb[0], bq);
        }
        __builtin_amdgcn_sched_barrier(0);
        // the wave issuing MFMAs goes first, so with two waves on a SIMD one
        // computes while the other waits on its loads
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          if (Cfg::SKIP && fm >= fm_act) continue;
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            if constexpr (Cfg::F8 && Cfg::WQ)  // B e2m1 (format 4) with its E8M0 block scale;
              // A scale 1, or 2^-4 for the second of two terms
              acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  fa[ks & 1][fm], fb[ks & 1][fn], acc[fm][fn], 0, 4, 0,
                  (Cfg::A2 && ks == 1) ? 127 - kTerm2Shift : 127, 0, scale_byte(fn, P, ks, ln));
            else if constexpr (Cfg::BS)  // this k-block's sums, scaled below
              tmp[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  fa[ks & 1][fm], fb[ks & 1][fn], ks == 0 ? f32x16{} : tmp[fm][fn], 0, 0, 0,
                  127, 0, 127);
            else if constexpr (Cfg::F8)
              acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  fa[ks & 1][fm], fb[ks & 1][fn], acc[fm][fn], 0, 0, 0, 127, 0, 127);
            else
              acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  fa[ks & 1][fm], fb[ks & 1][fn], acc[fm][fn], 0, 0, 0);
          }
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (Cfg::BS) {
        // the k-block's sums times their row and block scales (lane element i
        // is row 8 (i / 4) + 4 (lane / 32) + i % 4 of its fragment)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          if (Cfg::SKIP && fm >= fm_act) continue;
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            // (whole-vector updates keep the accumulators in registers)
            const float sw = __uint_as_float(bs_w[fn]);
            f32x16 s;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = __uint_as_float(bs_a[fm][i >> 2][i & 3]) * sw;
            acc[fm][fn] = acc[fm][fn] + tmp[fm][fn] * s;
          }
        }
      }
    };

    // prologue, in the order the wait model assumes
    load_scales(0);
    if constexpr (BKS == 1) {
      static_for<ST - 1>([&](auto s) {
#pragma unroll
        for (int p = 0; p < SUB; ++p) {
          gload_a(a_stage(s), c_stage(s), min(static_cast<int>(s), nk - 1), p);
          gload_b(b_stage(s), min(static_cast<int>(s), nk - 1), p);
        }
      });
    } else {
      static_for<SB - 1>([&](auto q) {
#pragma unroll
        for (int p = 0; p < SUB; ++p) gload_b(b_stage(q), min(static_cast<int>(q), nq - 1), p);
      });
      static_for<ST - 1>([&](auto s) {
#pragma unroll
        for (int p = 0; p < SUB; ++p)
          gload_a(a_stage(s), c_stage(s), min(static_cast<int>(s), nk - 1), p);
      });
    }
    wait_vmem<Cfg::WAIT_PRO>();
    stage_barrier();
    load_frags(lds_a0, lds_b0, opaque(lane), 0, 0, fa[0], fb[0], bq);

    // main loop, U k-steps per body, then the remaining k-steps
    int kt = 0;
    for (; kt + U <= nk; kt += U) static_for<U>([&](auto j) { kstep(j, kt + j); });
    static_for<U - 1>([&](auto j) {
      if (kt + j < nk) kstep(j, kt + j);
    });
    // No load of this tile may land in a stage after the next tile refills
    // it (each wave refills only the rows it loads itself).
    wait_vmem<0>();

    // epilogue: lane holds column (lane & 31) and rows 8*(i/4) + 4*(lane/32) + i%4
    // (from an opaque lane id: hoisted out of the tile loop, the 16 * FM row
    // indices would stay live across it)
    const int eln = opaque(lane);
    const int frag_row = eln & 31;
    const int frag_half = eln >> 5;
    // FP8: the products of codes times the row's activation scale and the
    // column's weight scale (per output channel; 0 past N_out, never stored)
    float sw[Cfg::F8 ? FN : 1];
    if constexpr (Cfg::F8 && !Cfg::WQ && !Cfg::BS) {
      const float* wsc = static_cast<const float*>(W_scales) + static_cast<int64_t>(e) * N_total;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int v = b_row0<Cfg>(wn, fn) + frag_row;
        const int col = Cfg::GATED ? (v < BN / 2 ? n0 + v : n0 + v - BN / 2) : n0 + v;
        sw[fn] = col < N_out ? wsc[wrow_of(v)] : 0.0f;
      }
    }
    auto scaled = [&](float a, float sa, int fn) -> float {
      if constexpr (Cfg::BS) return a;                  // scaled per k-block already
      if constexpr (Cfg::F8 && Cfg::WQ) return a * sa;  // block scales applied by the MFMA
      if constexpr (Cfg::F8) return a * sa * sw[fn];
      return a;
    };
    auto row_scale = [&](int r) -> float {
      if constexpr (Cfg::BS) return 1.0f;
      // (rows read from the tokens take their token's scale)
      if constexpr (Cfg::F8) return A_scales[gathered ? a_inv[row0 + r] / a_k : row0 + r];
      return 1.0f;
    };
    if (!Cfg::SPLIT && in_tail) {
      // fp32 sums of this piece into its slab, by virtual weight row (gated:
      // gate columns [0, BN/2), up columns [BN/2, BN)); piece 0 records the
      // tile's rows and columns for the reduction
      const int ti = tile - head_tiles;
      if (piece == 0 && tid == 0) {
        tail_hdr[2 + 3 * ti] = row0;
        tail_hdr[3 + 3 * ti] = min(rows, BM);  // rows of this tile (rows runs to the segment end)
        tail_hdr[4 + 3 * ti] = n0;
      }
      float* slab = reinterpret_cast<float*>(tail_ws + kTailHeader) +
                    static_cast<int64_t>(ti * St + piece) * (BM * BN);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        if (Cfg::SKIP && fm >= fm_act) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = wm * Cfg::WTM + fm * 32 + 8 * (i >> 2) + 4 * frag_half + (i & 3);
          if (r >= rows) continue;
          const float sa = row_scale(r);
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            slab[r * BN + b_row0<Cfg>(wn, fn) + frag_row] = scaled(acc[fm][fn][i], sa, fn);
        }
      }
      continue;
    }
    if (Cfg::SPLIT && S > 1) {
      // fp32 sums of this piece into slice `piece` (weight-row columns: gate
      // at n, up at N_out + n)
      float* P = partials + (static_cast<int64_t>(piece) * R_pad + row0) * N_total;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        if (Cfg::SKIP && fm >= fm_act) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = wm * Cfg::WTM + fm * 32 + 8 * (i >> 2) + 4 * frag_half + (i & 3);
          if (r >= rows) continue;
          float* prow = P + static_cast<int64_t>(r) * N_total;
          const float sa = row_scale(r);
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            const int v = b_row0<Cfg>(wn, fn) + frag_row;
            const int col = Cfg::GATED ? (v < BN / 2 ? n0 + v : n0 + v - BN / 2) : n0 + v;
            if (col < N_out) prow[wrow_of(v)] = scaled(acc[fm][fn][i], sa, fn);
          }
        }
      }
      continue;
    }
    // bf16 stores; the activation kind is a compile-time constant inside, so
    // the unrolled loops carry no branches on it
    auto store_tile = [&](auto kind) {
      constexpr int KIND = decltype(kind)::value;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        if (Cfg::SKIP && fm >= fm_act) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = wm * Cfg::WTM + fm * 32 + 8 * (i >> 2) + 4 * frag_half + (i & 3);
          if (r >= rows) continue;
          uint16_t* crow = C + static_cast<int64_t>(row0 + r) * N_out;
          const float sa = row_scale(r);
          if (Cfg::GATED) {
#pragma unroll
            for (int fn = 0; fn < FN / 2; ++fn) {
              const int col = n0 + wn * (Cfg::WTN / 2) + fn * 32 + frag_row;
              const float hv = gated_act_k<KIND>(scaled(acc[fm][fn][i], sa, fn),
                                                 scaled(acc[fm][fn + FN / 2][i], sa, fn + FN / 2),
                                                 cl);
              if (col < N_out) crow[col] = f32_to_bf16(hv);
            }
          } else {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
              const int col = n0 + wn * Cfg::WTN + fn * 32 + frag_row;
              if (col < N_out) crow[col] = f32_to_bf16(scaled(acc[fm][fn][i], sa, fn));
            }
          }
        }
      }
    };
    if constexpr (!Cfg::GATED) {
      store_tile(ic<0>{});
    } else {
      if (kind == 0) store_tile(ic<0>{});
      else if (kind == 1) store_tile(ic<1>{});
      else store_tile(ic<2>{});
    }
  }
}

// C[r, n] from the S fp32 slices: y = sum_s P[s, r, n], or for GEMM1
// h = act(sum_s P[s, r, n]) * sum_s P[s, r, I + n]; the slices are added in
// order s = 0, 1, ... (the same result on every run).  Rows at or past the
// local route count (past an expert's count in the batched experts format)
// are not written.  One thread per 4 output columns.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ partials,
                                                           const int* __restrict__ split,
                                                           const int32_t* __restrict__ offsets,
                                                           int E_l, int64_t R_pad, int N_out,
                                                           int gated, int act, float clamp,
                                                           int batch_m,
                                                           uint16_t* __restrict__ C) {
  const int S = split[0];
  if (S <= 1) return;
  const int64_t r = blockIdx.y;
  if (batch_m > 0) {
    const int e = static_cast<int>(r / batch_m);
    if (e >= E_l || r - static_cast<int64_t>(e) * batch_m >= min(max(offsets[e], 0), batch_m))
      return;
  } else if (r >= offsets[E_l]) {
    return;
  }
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (n >= N_out) return;
  const int N_total = gated ? 2 * N_out : N_out;
  const int64_t slice = R_pad * N_total;
  const float* p = partials + r * N_total + n;
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = gated ? *reinterpret_cast<const float4*>(p + N_out) : float4{};
  for (int s = 1; s < S; ++s) {
    const float4 x = *reinterpret_cast<const float4*>(p + s * slice);
    a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
    if (gated) {
      const float4 u = *reinterpret_cast<const float4*>(p + s * slice + N_out);
      b.x += u.x; b.y += u.y; b.z += u.z; b.w += u.w;
    }
  }
  if (gated) {
    const int kind = act_kind(act, clamp);
    const float cl = act_limit(clamp);
    auto f = [&](auto k) {
      constexpr int K = decltype(k)::value;
      a.x = gated_act_k<K>(a.x, b.x, cl);
      a.y = gated_act_k<K>(a.y, b.y, cl);
      a.z = gated_act_k<K>(a.z, b.z, cl);
      a.w = gated_act_k<K>(a.w, b.w, cl);
    };
    if (kind == 0) f(ic<0>{});
    else if (kind == 1) f(ic<1>{});
    else f(ic<2>{});
  }
  uint2 o;
  o.x = pack_bf16x2(a.x, a.y);
  o.y = pack_bf16x2(a.z, a.w);
  *reinterpret_cast<uint2*>(C + r * N_out + n) = o;
}

// The tail tiles from their slabs: C = sum over pieces s = 0, 1, ... of the
// slabs (fixed order), or for GEMM1 act(sum of gate) * (sum of up); block
// (i, y) covers part of tail tile i.  Tiles i >= the header's count exit.
__global__ __launch_bounds__(256) void tail_reduce_kernel(const char* __restrict__ ws, int BM,
                                                          int BN, int gated, int N_out, int act,
                                                          float clamp, uint16_t* __restrict__ C) {
  const int* hdr = reinterpret_cast<const int*>(ws);
  const int i = blockIdx.x;
  if (i >= hdr[0]) return;
  const int St = hdr[1];
  const int row0 = hdr[2 + 3 * i], rows = hdr[3 + 3 * i], n0 = hdr[4 + 3 * i];
  const int out_n = gated ? BN / 2 : BN;
  const int per_row = out_n / 4;
  const int64_t slab = static_cast<int64_t>(BM) * BN;
  const float* base = reinterpret_cast<const float*>(ws + kTailHeader) + i * St * slab;
  const int kind = act_kind(act, clamp);
  const float cl = act_limit(clamp);
  for (int idx = blockIdx.y * blockDim.x + threadIdx.x; idx < rows * per_row;
       idx += gridDim.y * blockDim.x) {
    const int r = idx / per_row;
    const int c = (idx - r * per_row) * 4;
    if (n0 + c >= N_out) continue;
    const float* p = base + static_cast<int64_t>(r) * BN + c;
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = gated ? *reinterpret_cast<const float4*>(p + out_n) : float4{};
    for (int sp = 1; sp < St; ++sp) {
      const float4 x = *reinterpret_cast<const float4*>(p + sp * slab);
      a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
      if (gated) {
        const float4 u = *reinterpret_cast<const float4*>(p + sp * slab + out_n);
        b.x += u.x; b.y += u.y; b.z += u.z; b.w += u.w;
      }
    }
    if (gated) {
      auto f = [&](auto kk) {
        constexpr int K = decltype(kk)::value;
        a.x = gated_act_k<K>(a.x, b.x, cl);
        a.y = gated_act_k<K>(a.y, b.y, cl);
        a.z = gated_act_k<K>(a.z, b.z, cl);
        a.w = gated_act_k<K>(a.w, b.w, cl);
      };
      if (kind == 0) f(ic<0>{});
      else if (kind == 1) f(ic<1>{});
      else f(ic<2>{});
    }
    uint2 o;
    o.x = pack_bf16x2(a.x, a.y);
    o.y = pack_bf16x2(a.z, a.w);
    *reinterpret_cast<uint2*>(C + static_cast<int64_t>(row0 + r) * N_out + n0 + c) = o;
  }
}

template <class Cfg>
hipError_t launch_cfg(const GemmArgs& g, int64_t max_rows, hipStream_t s) {
  static int occupancy = 0;
  if (occupancy == 0) {
    int occ = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, grouped_gemm_kernel<Cfg>,
                                                                Cfg::kThreads, 0);
    if (e != hipSuccess) return e;
    occupancy = occ > 0 ? occ : 1;
  }
  const int n_tiles = (g.N_out + Cfg::OUT_N - 1) / Cfg::OUT_N;
  const int64_t max_m = (max_rows + Cfg::BM - 1) / Cfg::BM + (g.E_l < max_rows ? g.E_l : max_rows);
  const int64_t max_tiles = max_m * n_tiles;
  int64_t grid = static_cast<int64_t>(device_cu_count()) * occupancy;
  if (grid > max_tiles) grid = max_tiles;
  if (grid >= 8) grid -= grid % 8;
  if (grid < 1) grid = 1;
  // split pieces: as many fp32 slices as the workspace holds (after a
  // 256-byte header that receives the chosen count), at most kMaxSplit
  const int64_t N_total = g.gated ? 2 * int64_t(g.N_out) : g.N_out;
  const int64_t slice_bytes = g.R_pad * N_total * int64_t(sizeof(float));
  int s_cap = 1;
  if (Cfg::SPLIT && g.split_ws != nullptr && slice_bytes > 0 && g.split_ws_bytes > kSplitHeader)
    s_cap = static_cast<int>(std::min<int64_t>(kMaxSplit, (g.split_ws_bytes - kSplitHeader) / slice_bytes));
  // (the reduce grid has one block row per permuted row: at most 65535)
  const bool split = s_cap >= 2 && g.N_out % 4 == 0 && g.R_pad <= 65535;
  int* hdr = split ? static_cast<int*>(g.split_ws) : nullptr;
  float* partials =
      split ? reinterpret_cast<float*>(static_cast<char*>(g.split_ws) + kSplitHeader) : nullptr;
  // tail split (tiles of the whole k-range): slabs of this tile in the scratch
  const int64_t slab_bytes = int64_t(Cfg::BM) * Cfg::BN * int64_t(sizeof(float));
  char* tail_ws = nullptr;
  int slab_cap = 0;
  if (!Cfg::SPLIT && g.split_ws != nullptr &&
      int64_t(g.split_ws_bytes) >= kTailHeader + 2 * slab_bytes) {
    tail_ws = static_cast<char*>(g.split_ws);
    slab_cap = static_cast<int>(
        std::min<int64_t>(kMaxTail * kMaxSplit, (int64_t(g.split_ws_bytes) - kTailHeader) / slab_bytes));
  }
  hipLaunchKernelGGL(grouped_gemm_kernel<Cfg>, dim3(static_cast<unsigned>(grid)),
                     dim3(Cfg::kThreads), 0, s,
                     g.a, g.w, g.w_scales, g.offsets, g.E_l, g.K,
                     g.N_out, g.R_pad, static_cast<uint16_t*>(g.c), n_tiles, partials, s_cap, hdr,
                     g.act, g.clamp, g.batch_m, g.a_scales, g.a_inv, g.a_k, g.a_T, tail_ws,
                     slab_cap, g.a_ld);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (tail_ws != nullptr) {
    hipLaunchKernelGGL(tail_reduce_kernel, dim3(kMaxTail, 8), dim3(256), 0, s, tail_ws, Cfg::BM,
                       Cfg::BN, g.gated, g.N_out, g.act, g.clamp, static_cast<uint16_t*>(g.c));
    return hipGetLastError();
  }
  if (!split) return e;
  const dim3 rgrid(static_cast<unsigned>((g.N_out / 4 + 255) / 256), static_cast<unsigned>(g.R_pad));
  hipLaunchKernelGGL(split_reduce_kernel, rgrid, dim3(256), 0, s, partials, hdr, g.offsets, g.E_l,
                     g.R_pad, g.N_out, g.gated, g.act, g.clamp, g.batch_m,
                     static_cast<uint16_t*>(g.c));
  return hipGetLastError();
}

template <bool WQ, bool F8, bool A2 = false, bool BS = false>
struct Configs {
  static constexpr int S3 = 3;  // activation stages of the 128-row tiles
  // The MFMA-bound 128x256 tile runs eight waves (4 x 2, a 32 x 128 block
  // each) in every format: with two waves per SIMD one computes while the
  // other waits on its loads.  Against four waves (2 x 2): bf16 5 % faster,
  // FP8 17 %, blockwise FP8 20 % (its k-block sums spill a few registers a
  // lane), FP8 or two-term activations with MXFP4 weights 4-22 %; MXFP4
  // weights with bf16 activations 50 times, since in four waves their 128
  // accumulators per lane beside the e2m1 expansion went to scratch.
  //                          BM   BN  WM WN ST  gated  WQ  GM  F8
  using Big   = TileCfg<128, 256, 4, 2, S3, false, WQ, 8, F8, A2, BS>;
  using BigG  = TileCfg<128, 256, 4, 2, S3, true, WQ, 8, F8, A2, BS>;
  using Wide  = TileCfg<128, 256, 1, 4, S3, false, WQ, 1, F8, A2, BS>;
  using WideG = TileCfg<128, 256, 1, 4, S3, true, WQ, 1, F8, A2, BS>;
  // the same tile in eight waves (2 x 4) when no split is possible: the
  // FP8 and MXFP4 weight streams gain from the second wave per SIMD (MXFP4
  // GEMM2 of the DeepSeek shape 12 % faster) what fragment skipping saves
  using WideP  = TileCfg<128, 256, 2, 4, S3, false, WQ, 1, F8, A2, BS>;
  using WidePG = TileCfg<128, 256, 2, 4, S3, true, WQ, 1, F8, A2, BS>;
  using Thin  = TileCfg<32, 256, 1, 4, 4, false, WQ, 8, F8, A2, BS>;
  using ThinG = TileCfg<32, 256, 1, 4, 4, true, WQ, 8, F8, A2, BS>;
};

// Tile shape from the mean rows per local expert (the host cannot see the
// real counts without a device round trip):
//   >= 128  MFMA-bound: the 128x256 tile, weight slices shared by GM m-tiles
//           (from 128 rows on it is 4-29 % faster than a 128x128 tile)
//   16-127  weight-streaming: one 128-row m-tile per expert, so every weight
//           byte is read once, with the idle fragments skipped
//   < 16    short tiles with split reductions (bf16: from 8 rows on the
//           weight-streaming tile, GEMM2 10-17 % faster than the short tile
//           there, GEMM1 level; FP8 and MXFP4 were level or slower); under 8
//           rows the whole-k decode kernels (bf16, per-channel FP8), which
//           from 8 to 15 rows the split tiles beat by up to 28 %.
constexpr int64_t kDecodeMeanRows = 8;

template <bool WQ, bool F8, bool A2 = false, bool BS = false>
hipError_t launch_fmt(const GemmArgs& g, int64_t max_rows, hipStream_t s) {
  using C = Configs<WQ, F8, A2, BS>;
  const int64_t mean_rows = g.E_l > 0 ? max_rows / g.E_l : max_rows;
  constexpr int64_t kThinMeanRows = (WQ || F8) ? 16 : 8;
  // bf16 decode batches: whole-k weight slices per workgroup, no split
  if constexpr (!WQ && !F8)
    if (mean_rows < kDecodeMeanRows && decode_gemm_fits(g)) return launch_decode_gemm(g, s);
  // FP8 decode batches (per-row and per-channel scales): the same, on FP8
  if constexpr (!WQ && F8 && !A2 && !BS)
    if (mean_rows < kDecodeMeanRows && decode_gemm_fp8_fits(g))
      return launch_decode_gemm_fp8(g, s);
  // can this call split its reductions (two fp32 slices in the workspace)?
  const int64_t slice = g.R_pad * (g.gated ? 2 * int64_t(g.N_out) : g.N_out) * 4;
  const bool may_split = g.split_ws != nullptr && g.R_pad <= 65535 &&
                         int64_t(g.split_ws_bytes) >= kSplitHeader + 2 * slice;
  // (FP8 x e2m1 GEMM1 streams fastest in four waves with fragment skipping)
  // (blockwise FP8 always: in the one-wave-row tile its four row fragments'
  // k-block sums and block scales beside the accumulators do not fit in
  // registers)
  const bool eight = BS || ((WQ || F8) && !may_split && !(WQ && F8 && g.gated));
  // (two-term activations, and MXFP4 weights with bf16 activations: always
  // the eight-wave tile in that range; with one wave row the doubled A
  // fragments, or the four row fragments beside the e2m1 expansion, do not
  // fit in registers, and the latter went to scratch, 30 times slower)
  constexpr bool always_eight = A2 || BS || (WQ && !F8);
  if (g.gated) {
    if (mean_rows >= 128) return launch_cfg<typename C::BigG>(g, max_rows, s);
    if (mean_rows >= kThinMeanRows) {
      if constexpr (always_eight) return launch_cfg<typename C::WidePG>(g, max_rows, s);
      else
        return eight ? launch_cfg<typename C::WidePG>(g, max_rows, s)
                     : launch_cfg<typename C::WideG>(g, max_rows, s);
    }
    return launch_cfg<typename C::ThinG>(g, max_rows, s);
  }
  if (mean_rows >= 128) return launch_cfg<typename C::Big>(g, max_rows, s);
  if (mean_rows >= kThinMeanRows) {
    if constexpr (always_eight) return launch_cfg<typename C::WideP>(g, max_rows, s);
    else
      return eight ? launch_cfg<typename C::WideP>(g, max_rows, s)
                   : launch_cfg<typename C::Wide>(g, max_rows, s);
  }
  return launch_cfg<typename C::Thin>(g, max_rows, s);
}

}  // namespace

size_t gemm_split_ws_bytes(int64_t R_pad, int N_total) {
  constexpr int64_t kBudget = int64_t(64) << 20;
  if (R_pad <= 0 || N_total <= 0) return 0;
  // split slices (few-row calls), or the tail split's slabs, whichever is larger
  int64_t split = 0;
  if (R_pad <= 65535) {
    const int64_t slice = R_pad * N_total * int64_t(sizeof(float));
    const int64_t n = std::min<int64_t>(kMaxSplit, kBudget / slice);
    split = n < 2 ? 0 : kSplitHeader + n * slice;
  }
  return static_cast<size_t>(std::max(split, kTailBytes));
}

bool gemm_picks_decode(const GemmArgs& g, int64_t max_rows) {
  const int64_t mean_rows = g.E_l > 0 ? max_rows / g.E_l : max_rows;
  return g.a_scales == nullptr && g.w_scales == nullptr && mean_rows < kDecodeMeanRows &&
         decode_gemm_fits(g);
}

// max_rows: the most local routes the call can see (T * k), from the host.
hipError_t launch_grouped_gemm(const GemmArgs& g, int64_t max_rows, hipStream_t s) {
  if (g.a_scales && g.a_ld > 0) return launch_fmt<false, true, false, true>(g, max_rows, s);
  if (g.a_scales && g.a_terms == 2) return launch_fmt<true, true, true>(g, max_rows, s);
  if (g.a_scales)
    return g.w_mxfp4 ? launch_fmt<true, true>(g, max_rows, s) : launch_fmt<false, true>(g, max_rows, s);
  return g.w_scales ? launch_fmt<true, false>(g, max_rows, s)
                    : launch_fmt<false, false>(g, max_rows, s);
}

}  // namespace moe
