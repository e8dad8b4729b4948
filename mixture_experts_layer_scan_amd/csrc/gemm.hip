// Grouped expert GEMMs (apply() of vLLM's modular fused-MoE kernel: GEMM1,
// the silu-and-mul activation, GEMM2, all unweighted).
//
//   C[r, n] = sum_k A[r, k] * W[e, n, k]     for r in expert e's row segment
//
// Both operands are contiguous along k, which is the natural operand layout
// of the CDNA4 MFMA v_mfma_f32_32x32x16_bf16 (each lane supplies 8 consecutive
// k of one row of A and of one row of W), so no transposes are needed.
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
// Tile pipeline (per k-step of BK, STAGES LDS stages)
//   - Operands move global -> LDS with buffer_load ... lds (16 bytes a lane,
//     straight into LDS, no registers): one wave instruction fills 1 KiB of a
//     stage.  Rows are stored XOR-swizzled in 16-byte chunks (swz below), the
//     lane choosing the global chunk the swizzle puts at its LDS position, so
//     MFMA operand reads are free of bank conflicts.
//   - k-step kt computes from stage kt % STAGES while the loads of k-step
//     kt + STAGES - 1 stream into the stage computed one k-step earlier.  A
//     k-step ends by waiting until this wave's loads of k-step kt + 1 landed
//     (a partial vmcnt: later k-steps stay in flight) and a barrier, so global
//     latency is hidden behind STAGES - 1 k-steps of MFMAs.
//   - Inside a k-step, fenced so the compiler keeps the order: the operand
//     reads of sub-step ks + 1 and a slice of the loads are issued before the
//     MFMAs of sub-step ks.
//
// MXFP4 weights (e2m1 pairs, low nibble = even k, one E8M0 scale byte per 32
// k; vLLM flashinfer_moe_ep.py, _E2M1_LUT and _dequant_fp4_ue8m0_gran32): the
// packed tile (32 bytes per row per k-step) is loaded into LDS the same way;
// each lane reads its 16 bytes once per k-step and expands 4 of them per
// sub-step to bf16 with v_cvt_scalef32_pk_bf16_fp4 (value x 2^(s-127), exact
// in bf16), so the MFMAs and the activations stay bf16.  Inside a k-step,
// sub-step ks and lane half h cover k = 32h + 8ks .. +7 for A and W alike,
// which makes a lane's packed bytes of one k-step contiguous and puts all its
// k in one 32-wide scale block.
//
// GEMM1 ("gated"): a tile of BN virtual weight rows holds BN/2 gate rows
// [n0, n0 + BN/2) and the matching BN/2 up rows [I + n0, ...).  Each wave
// computes gate and up blocks with the same lane layout, so the epilogue
// forms silu(g) * u in registers and writes BN/2 columns of h.
#include "moe_common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Descriptor word 3 for raw (untyped, stride 0) buffer access on gfx9-family
// parts: 32-bit data format, out-of-range offsets read as zero.
constexpr int kBufferFlags = 0x00020000;

// Swizzle of 16-byte chunk positions within a tile row of BK bf16:
//   BK = 64 (8 chunks, 128-byte rows): chunk c of row r sits at
//           c ^ (r & 7) ^ ((r >> 3) & 1);
//   BK = 32 (4 chunks, 64-byte rows):  c ^ ((r >> 2) & 3).
// Either way 16 consecutive rows read at one logical chunk (a 16-lane group
// of an MFMA operand read) hit 16 distinct 16-byte bank groups of the 64-bank
// LDS.
template <int BK>
__device__ __forceinline__ int swz_key(int row) {
  if constexpr (BK == 64) return (row & 7) ^ ((row >> 3) & 1);
  else return (row >> 2) & 3;
}

template <int BK>
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ swz_key<BK>(row)) << 3);
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

template <int BM_, int BN_, int WM_, int WN_, int BK_, int STAGES_, bool GATED_, bool WQ_ = false,
          int GM_ = 8>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, STAGES = STAGES_;
  static constexpr bool GATED = GATED_;
  static constexpr bool WQ = WQ_;  // weights in MXFP4
  static constexpr int GM = GM_;   // m-tiles per group of the tile order
  static constexpr int NWAVES = WM * WN;
  static constexpr int kThreads = NWAVES * kWave;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  // skip row fragments past the segment (one wave row only: otherwise the
  // waves of the lower rows would idle while the others work)
  static constexpr bool SKIP = (WM == 1 && FM > 1);
  static constexpr int CHUNKS = BK / 8;               // 16-byte chunks per tile row
  static constexpr int ROWS_PER_LD = kWave / CHUNKS;  // tile rows per 1 KiB load
  static constexpr int A_LD = BM / ROWS_PER_LD / NWAVES;  // loads per wave per k-step
  // MXFP4: a packed row of one k-step is 32 bytes, so one load covers 32 rows
  static constexpr int B_LD = WQ ? BN / 32 / NWAVES : BN / ROWS_PER_LD / NWAVES;
  static constexpr int SUBSTEPS = BK / 16;
  static constexpr int OUT_N = GATED ? BN / 2 : BN;
  static constexpr int A_ELEMS = BM * BK;                  // uint16 units
  static constexpr int B_ELEMS = WQ ? BN * 16 : BN * BK;   // uint16 units (packed: 32 B/row)
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  // vector-memory loads per wave per k-step: tile loads (+ one scale byte per
  // weight fragment for MXFP4)
  static constexpr int LOADS = A_LD + B_LD + (WQ ? FN : 0);
  // Loads a wave may leave in flight at the end of a k-step so that those of
  // the next k-step have landed.  In steady state that is (STAGES - 2) * LOADS;
  // the prologue issues no scale loads between its tile loads, so the first
  // k-steps need the smaller count below (it also covers the steady state: the
  // extra scale loads it waits for were consumed a k-step earlier anyway).
  static constexpr int WAIT = (STAGES - 2) * (A_LD + B_LD) + ((WQ && STAGES > 2) ? FN : 0);
  static_assert(BK == 32 || BK == 64, "k-step");
  static_assert(!WQ || BK == 64, "MXFP4 tiles use 64-wide k-steps (two scale blocks)");
  static_assert(STAGES >= 2 && STAGES <= 4, "stages");
  static_assert(WAIT < 64, "in-flight loads must fit vmcnt");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(!GATED || (FN % 2 == 0), "gated tiles pair gate and up blocks");
  static_assert(BM % (ROWS_PER_LD * NWAVES) == 0 && BN % ((WQ ? 32 : ROWS_PER_LD) * NWAVES) == 0,
                "whole load instructions");
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

// E8M0 scale byte -> the float whose bit pattern is s << 23 (2^(s-127);
// s = 0 gives 0, s = 255 gives +inf).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) { return __uint_as_float(s << 23); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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
    const uint16_t* __restrict__ A, const void* __restrict__ W,
    const uint8_t* __restrict__ W_scales, const int32_t* __restrict__ offsets, int E_l, int K,
    int N_out, int64_t R_pad, uint16_t* __restrict__ C, int n_tiles) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, FM = Cfg::FM, FN = Cfg::FN;
  constexpr int NT = Cfg::kThreads, ST = Cfg::STAGES, SUB = Cfg::SUBSTEPS;
  // LDS stages as distinct objects, so the compiler knows that loads into one
  // never alias operand reads from another (unused ones are tiny)
  __shared__ __attribute__((aligned(16))) uint16_t lds_s0[Cfg::STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t lds_s1[Cfg::STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t lds_s2[ST > 2 ? Cfg::STAGE : 8];
  __shared__ __attribute__((aligned(16))) uint16_t lds_s3[ST > 3 ? Cfg::STAGE : 8];
  __shared__ int32_t s_mt[1025];
  __shared__ int32_t s_scratch[16];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;

  // m-tile numbering: s_mt[e] = m-tiles of experts < e.
  {
    const int per = (E_l + NT - 1) / NT;
    int local = 0;
    for (int i = 0; i < per; ++i) {
      const int e = tid * per + i;
      if (e < E_l) local += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
    }
    int total_m = 0;
    int run = block_exclusive_sum(local, s_scratch, &total_m);
    for (int i = 0; i < per; ++i) {
      const int e = tid * per + i;
      if (e < E_l) {
        s_mt[e] = run;
        run += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
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
  const int nk = K / BK;

  // Load j of this wave fills tile rows [R rb, R rb + R) (R = ROWS_PER_LD,
  // rb = j * NWAVES + wave); lane L writes the 16 bytes at LDS row
  // R rb + L / CHUNKS, position L % CHUNKS, so it fetches the logical chunk
  // the swizzle puts there.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int ld_sub = lane / Cfg::CHUNKS;
  const int ld_pos = lane % Cfg::CHUNKS;

  for (int tile = slot; tile < total_tiles; tile += G) {
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
    const int e = lo;
    const int seg_end = min(static_cast<int64_t>(offsets[e + 1]), R_pad);
    const int row0 = offsets[e] + (m_tile - s_mt[e]) * BM;
    const int rows = seg_end - row0;
    if (rows <= 0) continue;
    const int n0 = n_tile * Cfg::OUT_N;
    // row fragments of this wave that hold rows of the segment (wave-uniform)
    const int fm_act = Cfg::SKIP ? min(FM, (rows - wm * Cfg::WTM + 31) / 32) : FM;

    // Buffer descriptors: A over rows [row0, seg_end) of this expert, W over
    // this expert's weights; loads past either range return zero.
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(A + static_cast<int64_t>(row0) * K), 0,
        static_cast<int>(static_cast<uint32_t>(rows) * static_cast<uint32_t>(K) * 2u),
        kBufferFlags);
    // weight bytes per row: K * 2 (bf16) or K / 2 (packed e2m1)
    const uint32_t w_row_bytes = Cfg::WQ ? static_cast<uint32_t>(K) / 2u : static_cast<uint32_t>(K) * 2u;
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(W) +
                             static_cast<int64_t>(e) * N_total * w_row_bytes),
        0, static_cast<int>(static_cast<uint32_t>(N_total) * w_row_bytes), kBufferFlags);
    uint32_t a_off[Cfg::A_LD];
#pragma unroll
    for (int j = 0; j < Cfg::A_LD; ++j) {
      const int r = (j * Cfg::NWAVES + wave_u) * Cfg::ROWS_PER_LD + ld_sub;
      const int c = ld_pos ^ swz_key<BK>(r);
      a_off[j] = (static_cast<uint32_t>(r) * K + c * 8) * 2u;
    }
    // gated: virtual rows [0, BN/2) are gate rows n0 + v, the rest up rows
    // I + n0 + v - BN/2; columns past N_out are loaded but never stored
    auto wrow_of = [&](int v) {
      return Cfg::GATED ? (v < BN / 2 ? n0 + v : N_out + n0 + v - BN / 2) : n0 + v;
    };
    uint32_t b_off[Cfg::B_LD];
#pragma unroll
    for (int j = 0; j < Cfg::B_LD; ++j) {
      if constexpr (Cfg::WQ) {
        // 32 rows per load, lane L -> row L / 2, 16-byte position L % 2
        const int v = (j * Cfg::NWAVES + wave_u) * 32 + (lane >> 1);
        const int c = (lane & 1) ^ ((v >> 3) & 1);
        b_off[j] = static_cast<uint32_t>(wrow_of(v)) * w_row_bytes + c * 16;
      } else {
        const int v = (j * Cfg::NWAVES + wave_u) * Cfg::ROWS_PER_LD + ld_sub;
        const int c = ld_pos ^ swz_key<BK>(v);
        b_off[j] = static_cast<uint32_t>(wrow_of(v)) * w_row_bytes + c * 16;
      }
    }
    // MXFP4 scale bytes: lane's weight row per fragment, block 2 kt + half
    const uint32_t s_row = Cfg::WQ ? static_cast<uint32_t>(K) / 32u : 0u;  // scale bytes per row
    const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(W_scales + static_cast<int64_t>(e) * N_total * s_row), 0,
        static_cast<int>(static_cast<uint32_t>(N_total) * s_row), kBufferFlags);
    uint32_t s_off[Cfg::WQ ? FN : 1];
    uint32_t sc_cur[Cfg::WQ ? FN : 1], sc_nxt[Cfg::WQ ? FN : 1];
    if constexpr (Cfg::WQ) {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        s_off[fn] = static_cast<uint32_t>(wrow_of(b_row0<Cfg>(wn, fn) + (lane & 31))) * s_row +
                    (lane >> 5);
    }
    auto load_scales = [&](uint32_t* dst, int kt) {
      if constexpr (Cfg::WQ) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) dst[fn] = load_byte(s_rsrc, s_off[fn], kt * 2);
      }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    // Slice `part` (of SUB) of k-step kt of A and W into LDS stage `st`: the
    // loads of one k-step are spread over its sub-steps.
    auto gload = [&](uint16_t* st, int kt, int part) {
      const int soff = kt * BK * 2;
      const int soff_b = Cfg::WQ ? kt * BK / 2 : soff;
#pragma unroll
      for (int j = 0; j < Cfg::A_LD; ++j)
        if (j % SUB == part)
          lds_dma16(a_rsrc, st + (j * Cfg::NWAVES + wave_u) * Cfg::ROWS_PER_LD * BK, a_off[j],
                    soff);
#pragma unroll
      for (int j = 0; j < Cfg::B_LD; ++j)
        if ((j + Cfg::A_LD) % SUB == part)
          lds_dma16(b_rsrc, st + Cfg::A_ELEMS + (j * Cfg::NWAVES + wave_u) * 512, b_off[j],
                    soff_b);
    };
    auto gload_all = [&](uint16_t* st, int kt) {
#pragma unroll
      for (int p = 0; p < SUB; ++p) gload(st, kt, p);
    };

    // Operand fragments of k sub-step ks from stage `as`: lane half h holds
    // k = 32h + 8ks .. +7 of its A row and of its W row.  `ln` is the lane id
    // made opaque per k-step so the (swizzled) addresses are rebuilt there
    // instead of all being kept live.  MXFP4: at ks == 0 the lane's 16 packed
    // bytes of the k-step are read into `bq`; every sub-step expands 4 of them.
    auto load_frags = [&](const uint16_t* as, int ln, int ks, bf16x8* af, bf16x8* bfr, uint4* bq,
                          const uint32_t* sc) {
      const uint16_t* bs = as + Cfg::A_ELEMS;
      const int frag_row = ln & 31;
      const int half = ln >> 5;
      const int chunk = half * SUB + ks;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        if (Cfg::SKIP && fm > 0 && fm >= fm_act) continue;
        const int r = wm * Cfg::WTM + fm * 32 + frag_row;
        af[fm] = *reinterpret_cast<const bf16x8*>(as + swz<BK>(r, chunk));
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int v = b_row0<Cfg>(wn, fn) + frag_row;
        if constexpr (Cfg::WQ) {
          if (ks == 0) bq[fn] = *reinterpret_cast<const uint4*>(bs + v * 16 + ((half ^ ((v >> 3) & 1)) << 3));
          const uint32_t word = ks == 0 ? bq[fn].x : ks == 1 ? bq[fn].y : ks == 2 ? bq[fn].z : bq[fn].w;
          bfr[fn] = expand_fp4x8(word, e8m0_to_f32(sc[fn]));
        } else {
          bfr[fn] = *reinterpret_cast<const bf16x8*>(bs + swz<BK>(v, chunk));
        }
      }
    };

    // Operand fragments, double-buffered by sub-step; buffer 0 holds sub-step
    // 0 of the next k-step when a k-step begins.
    static_assert(SUB % 2 == 0, "sub-step 0 of the next k-step reuses buffer 0");
    bf16x8 fa[2][FM], fb[2][FN];
    uint4 bq[Cfg::WQ ? FN : 1];

    // k-step kt from stage `cur` while k-step kt + ST - 1 streams into `ld`
    // (the stage computed in the previous k-step, which the barrier closed);
    // the last k-steps reload the final one into stages nobody reads again.
    // The barrier that closes `cur` and opens `nxt` (k-step kt + 1) comes
    // before the last sub-step's MFMAs, and sub-step 0 of `nxt` is read right
    // after it, so that LDS latency hides behind those MFMAs.
    auto kstep = [&](const uint16_t* cur, const uint16_t* nxt, uint16_t* ld, int kt) {
      const int kn = min(kt + ST - 1, nk - 1);
      load_scales(sc_nxt, min(kt + 1, nk - 1));  // before the tile loads: see the vmcnt count
      const int ln = opaque(lane);
#pragma unroll
      for (int ks = 0; ks < SUB; ++ks) {
        if (ks + 1 < SUB) load_frags(cur, ln, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1], bq, sc_cur);
        gload(ld, kn, ks);
        if (ks + 1 == SUB) {
          // this wave's loads of k-step kt + 1 landed and its reads of `cur`
          // returned; after the barrier, every wave's have
          wait_vmem_lds<Cfg::WAIT>();
          stage_barrier();
          load_frags(nxt, ln, 0, fa[0], fb[0], bq, sc_nxt);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          if (Cfg::SKIP && fm > 0 && fm >= fm_act) continue;
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks & 1][fm], fb[ks & 1][fn],
                                                                  acc[fm][fn], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (Cfg::WQ) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) sc_cur[fn] = sc_nxt[fn];
      }
    };

    // prologue: scales of k-step 0, k-steps 0 .. ST-2 in flight, then k-step 0
    // complete (the prologue issues no scale loads after the tile loads)
    load_scales(sc_cur, 0);
    gload_all(lds_s0, 0);
    if constexpr (ST > 2) gload_all(lds_s1, min(1, nk - 1));
    if constexpr (ST > 3) gload_all(lds_s2, min(2, nk - 1));
    wait_vmem<(ST - 2) * (Cfg::A_LD + Cfg::B_LD)>();
    stage_barrier();
    load_frags(lds_s0, opaque(lane), 0, fa[0], fb[0], bq, sc_cur);

    // main loop unrolled by ST, so every stage is a compile-time object:
    // k-step kt reads stage kt % ST, opens (kt + 1) % ST and loads into
    // stage (kt - 1) % ST
    int kt = 0;
    if constexpr (ST == 2) {
      for (; kt + 1 < nk; kt += 2) {
        kstep(lds_s0, lds_s1, lds_s1, kt);
        kstep(lds_s1, lds_s0, lds_s0, kt + 1);
      }
      if (kt < nk) kstep(lds_s0, lds_s1, lds_s1, kt);
    } else if constexpr (ST == 3) {
      for (; kt + 2 < nk; kt += 3) {
        kstep(lds_s0, lds_s1, lds_s2, kt);
        kstep(lds_s1, lds_s2, lds_s0, kt + 1);
        kstep(lds_s2, lds_s0, lds_s1, kt + 2);
      }
      if (kt < nk) kstep(lds_s0, lds_s1, lds_s2, kt);
      if (kt + 1 < nk) kstep(lds_s1, lds_s2, lds_s0, kt + 1);
    } else {
      for (; kt + 3 < nk; kt += 4) {
        kstep(lds_s0, lds_s1, lds_s3, kt);
        kstep(lds_s1, lds_s2, lds_s0, kt + 1);
        kstep(lds_s2, lds_s3, lds_s1, kt + 2);
        kstep(lds_s3, lds_s0, lds_s2, kt + 3);
      }
      if (kt < nk) kstep(lds_s0, lds_s1, lds_s3, kt);
      if (kt + 1 < nk) kstep(lds_s1, lds_s2, lds_s0, kt + 1);
      if (kt + 2 < nk) kstep(lds_s2, lds_s3, lds_s1, kt + 2);
    }
    // No load of this tile may land in a stage after the next tile refills
    // it (each wave refills only the rows it loads itself).
    wait_vmem<0>();

    const int frag_row = lane & 31;
    const int frag_half = lane >> 5;
    // epilogue: lane holds column (lane & 31) and rows 8*(i/4) + 4*(lane/32) + i%4
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (Cfg::SKIP && fm > 0 && fm >= fm_act) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = wm * Cfg::WTM + fm * 32 + 8 * (i >> 2) + 4 * frag_half + (i & 3);
        if (r >= rows) continue;
        uint16_t* crow = C + static_cast<int64_t>(row0 + r) * N_out;
        if (Cfg::GATED) {
#pragma unroll
          for (int fn = 0; fn < FN / 2; ++fn) {
            const int col = n0 + wn * (Cfg::WTN / 2) + fn * 32 + frag_row;
            const float g = acc[fm][fn][i];
            const float u = acc[fm][fn + FN / 2][i];
            const float hv = g / (1.0f + __expf(-g)) * u;
            if (col < N_out) crow[col] = f32_to_bf16(hv);
          }
        } else {
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            const int col = n0 + wn * Cfg::WTN + fn * 32 + frag_row;
            if (col < N_out) crow[col] = f32_to_bf16(acc[fm][fn][i]);
          }
        }
      }
    }
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
  hipLaunchKernelGGL(grouped_gemm_kernel<Cfg>, dim3(static_cast<unsigned>(grid)),
                     dim3(Cfg::kThreads), 0, s,
                     static_cast<const uint16_t*>(g.a), g.w, g.w_scales, g.offsets, g.E_l, g.K,
                     g.N_out, g.R_pad, static_cast<uint16_t*>(g.c), n_tiles);
  return hipGetLastError();
}

template <bool WQ>
struct Configs {
  //                          BM   BN  WM WN  BK ST  gated      GM
  using Big   = TileCfg<128, 256, 2, 2, 64, 3, false, WQ>;
  using BigG  = TileCfg<128, 256, 2, 2, 64, 3, true, WQ>;
  using Mid   = TileCfg<128, 128, 2, 2, 64, 2, false, WQ>;
  using MidG  = TileCfg<128, 128, 2, 2, 64, 2, true, WQ>;
  using Wide  = TileCfg<128, 256, 1, 4, 64, 3, false, WQ, 1>;
  using WideG = TileCfg<128, 256, 1, 4, 64, 3, true, WQ, 1>;
  using Thin  = TileCfg<32, 256, 1, 4, 64, 4, false, WQ>;
  using ThinG = TileCfg<32, 256, 1, 4, 64, 4, true, WQ>;
};

// Tile shape from the mean rows per local expert (the host cannot see the
// real counts without a device round trip):
//   >= 128  MFMA-bound: square-ish tiles, weight slices shared by GM m-tiles
//   16-127  weight-streaming: one 128-row m-tile per expert, so every weight
//           byte is read once, with the idle fragments skipped
//   < 16    decode: short tiles.
template <bool WQ>
hipError_t launch_fmt(const GemmArgs& g, int64_t max_rows, hipStream_t s) {
  using C = Configs<WQ>;
  const int64_t mean_rows = g.E_l > 0 ? max_rows / g.E_l : max_rows;
  if (g.gated) {
    if (mean_rows >= 512) return launch_cfg<typename C::BigG>(g, max_rows, s);
    if (mean_rows >= 128) return launch_cfg<typename C::MidG>(g, max_rows, s);
    if (mean_rows >= 16) return launch_cfg<typename C::WideG>(g, max_rows, s);
    return launch_cfg<typename C::ThinG>(g, max_rows, s);
  }
  if (mean_rows >= 512) return launch_cfg<typename C::Big>(g, max_rows, s);
  if (mean_rows >= 128) return launch_cfg<typename C::Mid>(g, max_rows, s);
  if (mean_rows >= 16) return launch_cfg<typename C::Wide>(g, max_rows, s);
  return launch_cfg<typename C::Thin>(g, max_rows, s);
}

}  // namespace

// max_rows: the most local routes the call can see (T * k), from the host.
hipError_t launch_grouped_gemm(const GemmArgs& g, int64_t max_rows, hipStream_t s) {
  return g.w_scales ? launch_fmt<true>(g, max_rows, s) : launch_fmt<false>(g, max_rows, s);
}

}  // namespace moe
