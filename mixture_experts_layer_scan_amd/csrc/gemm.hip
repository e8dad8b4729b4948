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
//     groups of GROUP_M m-tiles per n-tile column, so the tiles one XCD runs
//     together share A rows and weight rows in that XCD's L2.
//   - Loads go through buffer descriptors bounded to the expert's row segment
//     and to the expert's weights: rows of a ragged m-tile past the segment
//     read as zero (never another expert's rows) and are masked on store.
//
// Tile pipeline: BK = 64 (one 128-byte row per operand row), two LDS stages.
// Each thread moves 16-byte chunks; chunk c of tile row r lives at chunk
// c ^ (r & 7) of that row, which spreads the MFMA operand reads (32 rows, same
// chunk) over the LDS banks.  The next stage's global loads are issued before
// the current stage's MFMAs and stored to the other LDS buffer after them:
// one barrier per k-step.
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

constexpr int BK = 64;
constexpr int GROUP_M = 8;

// Descriptor word 3 for raw (untyped, stride 0) buffer access on gfx9-family
// parts: 32-bit data format, out-of-range offsets read as zero.
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), soff, 0);
  return uint4{v[0], v[1], v[2], v[3]};
}

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ (row & 7)) << 3);
}

template <int BM_, int BN_, int WM_, int WN_, bool GATED_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr bool GATED = GATED_;
  static constexpr int kThreads = WM * WN * kWave;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int ROWS_PER_PASS = kThreads / 8;  // tile rows loaded per chunk pass
  static constexpr int A_CH = BM / ROWS_PER_PASS;
  static constexpr int B_CH = BN / ROWS_PER_PASS;
  static constexpr int OUT_N = GATED ? BN / 2 : BN;
  static constexpr int STAGE = (BM + BN) * BK;  // bf16 elements per LDS stage
  static constexpr size_t LDS_BYTES = 2 * STAGE * sizeof(uint16_t);
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(!GATED || (FN % 2 == 0), "gated tiles pair gate and up blocks");
  static_assert(BM % ROWS_PER_PASS == 0 && BN % ROWS_PER_PASS == 0, "load passes");
};

template <class Cfg>
__global__ __launch_bounds__(Cfg::kThreads) void grouped_gemm_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
    const int32_t* __restrict__ offsets, int E_l, int K, int N_out, int64_t R_pad,
    uint16_t* __restrict__ C, int n_tiles) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, FM = Cfg::FM, FN = Cfg::FN;
  constexpr int NT = Cfg::kThreads;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
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

  const int ld_row = tid >> 3;  // tile row of this thread's first chunk
  const int ld_chunk = tid & 7;
  const int ld_lds = swz(ld_row, ld_chunk);  // + i * ROWS_PER_PASS * BK for pass i

  for (int tile = slot; tile < total_tiles; tile += G) {
    // grouped order: GROUP_M m-tiles share each n-tile column
    const int group = GROUP_M * n_tiles;
    const int gid = tile / group;
    const int first_m = gid * GROUP_M;
    const int gm = min(total_m - first_m, GROUP_M);
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

    // Global sources through buffer descriptors: the A descriptor covers the
    // rows [row0, seg_end) of this expert and the W descriptor this expert's
    // weights, so a load past either range returns zero and never touches
    // other memory.  Per-thread byte offsets stay fixed over the k loop; the
    // k-step goes into the scalar offset.
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(A + static_cast<int64_t>(row0) * K), 0,
        static_cast<int>(static_cast<uint32_t>(rows) * static_cast<uint32_t>(K) * 2u), kBufferFlags);
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(W + static_cast<int64_t>(e) * N_total * K), 0,
        static_cast<int>(static_cast<uint32_t>(N_total) * static_cast<uint32_t>(K) * 2u), kBufferFlags);
    uint32_t a_off[Cfg::A_CH];
#pragma unroll
    for (int i = 0; i < Cfg::A_CH; ++i)
      a_off[i] = (static_cast<uint32_t>(ld_row + i * Cfg::ROWS_PER_PASS) * K + ld_chunk * 8) * 2u;
    uint32_t b_off[Cfg::B_CH];
#pragma unroll
    for (int i = 0; i < Cfg::B_CH; ++i) {
      const int v = ld_row + i * Cfg::ROWS_PER_PASS;
      // gated: virtual rows [0, BN/2) are gate rows n0 + v, the rest up rows
      // I + n0 + v - BN/2; columns past N_out are loaded but never stored
      const int wrow = Cfg::GATED ? (v < BN / 2 ? n0 + v : N_out + n0 + v - BN / 2) : n0 + v;
      b_off[i] = (static_cast<uint32_t>(wrow) * K + ld_chunk * 8) * 2u;
    }

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    uint4 ra[Cfg::A_CH], rb[Cfg::B_CH];
    auto gload = [&](int kt) {
#pragma unroll
      for (int i = 0; i < Cfg::A_CH; ++i) ra[i] = bload(a_rsrc, a_off[i], kt * BK * 2);
#pragma unroll
      for (int i = 0; i < Cfg::B_CH; ++i) rb[i] = bload(b_rsrc, b_off[i], kt * BK * 2);
    };
    auto sstore = [&](int stage) {
      uint16_t* as = lds + stage * Cfg::STAGE;
      uint16_t* bs = as + BM * BK;
#pragma unroll
      for (int i = 0; i < Cfg::A_CH; ++i)
        *reinterpret_cast<uint4*>(as + ld_lds + i * Cfg::ROWS_PER_PASS * BK) = ra[i];
#pragma unroll
      for (int i = 0; i < Cfg::B_CH; ++i)
        *reinterpret_cast<uint4*>(bs + ld_lds + i * Cfg::ROWS_PER_PASS * BK) = rb[i];
    };

    const int frag_row = lane & 31;
    const int frag_half = lane >> 5;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) gload(kt + 1);
      const uint16_t* as = lds + cur * Cfg::STAGE;
      const uint16_t* bs = as + BM * BK;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int chunk = ks * 2 + frag_half;
        bf16x8 af[FM], bfr[FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          const int r = wm * Cfg::WTM + fm * 32 + frag_row;
          af[fm] = *reinterpret_cast<const bf16x8*>(as + swz(r, chunk));
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          int v;
          if (Cfg::GATED) {
            v = (fn < FN / 2) ? wn * (Cfg::WTN / 2) + fn * 32
                              : BN / 2 + wn * (Cfg::WTN / 2) + (fn - FN / 2) * 32;
          } else {
            v = wn * Cfg::WTN + fn * 32;
          }
          bfr[fn] = *reinterpret_cast<const bf16x8*>(bs + swz(v + frag_row, chunk));
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
      }
      if (kt + 1 < nk) sstore(cur ^ 1);
      __syncthreads();
    }

    // epilogue: lane holds column (lane & 31) and rows 8*(i/4) + 4*(lane/32) + i%4
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
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
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(grouped_gemm_kernel<Cfg>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(Cfg::LDS_BYTES));
    if (e != hipSuccess) return e;
    int occ = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, grouped_gemm_kernel<Cfg>,
                                                     Cfg::kThreads, Cfg::LDS_BYTES);
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
                     dim3(Cfg::kThreads), Cfg::LDS_BYTES, s,
                     static_cast<const uint16_t*>(g.a), static_cast<const uint16_t*>(g.w),
                     g.offsets, g.E_l, g.K, g.N_out, g.R_pad, static_cast<uint16_t*>(g.c),
                     n_tiles);
  return hipGetLastError();
}

using Big = TileCfg<256, 256, 2, 2, false>;
using BigG = TileCfg<256, 256, 2, 2, true>;
using Mid = TileCfg<128, 128, 2, 2, false>;
using MidG = TileCfg<128, 128, 2, 2, true>;
using Slim = TileCfg<64, 256, 1, 4, false>;
using SlimG = TileCfg<64, 256, 1, 4, true>;
using Thin = TileCfg<32, 256, 1, 4, false>;
using ThinG = TileCfg<32, 256, 1, 4, true>;

}  // namespace

// max_rows: the most local routes the call can see (T * k), from the host.
// Tile height follows the mean rows per local expert (the host cannot see the
// real counts without a device round trip).
hipError_t launch_grouped_gemm(const GemmArgs& g, int64_t max_rows, hipStream_t s) {
  const int64_t mean_rows = g.E_l > 0 ? max_rows / g.E_l : max_rows;
  if (g.gated) {
    if (mean_rows >= 512) return launch_cfg<BigG>(g, max_rows, s);
    if (mean_rows >= 128) return launch_cfg<MidG>(g, max_rows, s);
    if (mean_rows >= 48) return launch_cfg<SlimG>(g, max_rows, s);
    return launch_cfg<ThinG>(g, max_rows, s);
  }
  if (mean_rows >= 512) return launch_cfg<Big>(g, max_rows, s);
  if (mean_rows >= 128) return launch_cfg<Mid>(g, max_rows, s);
  if (mean_rows >= 48) return launch_cfg<Slim>(g, max_rows, s);
  return launch_cfg<Thin>(g, max_rows, s);
}

}  // namespace moe
