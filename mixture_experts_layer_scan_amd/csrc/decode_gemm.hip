// Grouped GEMM for decode batches (bf16): the [Experts] GEMMs of vLLM's
// modular fused-MoE kernel (apply(): GEMM1 with act(gate) * up, GEMM2) when
// each local expert receives only a few rows.
//
// With a handful of rows per expert the GEMMs are weight streams: every
// weight byte is read once and each feeds a few multiply-adds.  The tiled
// kernel then needs a split reduction to give every compute unit a share of
// one expert's weights, and each share is too short to fill its load
// pipeline.  Here a work item is a slice of 16 weight rows of one expert over
// the whole k-range (for GEMM1: 8 gate rows and the 8 matching up rows), so a
// workgroup streams one long run of each row and no reduction kernel follows:
//   - 8 waves split the k-range; lane l streams 16 contiguous bytes of weight
//     row l % 16 per 32-k step (four lanes cover a row's 64-byte run), with
//     4 steps of loads in flight (one when the range is not a multiple of 4
//     steps), and two workgroups share a compute unit;
//   - a workgroup's work units (item, pass of 16 rows) follow one another
//     without a pipeline drain: the next unit's first loads are issued
//     before the current unit's last MFMAs, reduction and stores;
//   - the 16 x 16 x 32 bf16 MFMA takes the expert's rows (up to 16 per pass)
//     as A and the 16 weight rows as B, so the sum over k happens in the
//     matrix core and each lane keeps four fp32 sums;
//   - the 8 waves' sums add up in LDS; GEMM1 pairs gate column j with up
//     column j + 8 through a lane shuffle and applies the activation.
// Rows come from the permuted activations, or (gathered form) from the token
// rows through the permute's inverse map.  An expert with more than 16 rows
// takes one pass per 16 (each pass re-reads the slice), so the host picks
// this kernel only for batches whose experts see a few rows each.
#include "route_core.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * kWave;
constexpr int kDecRows = 16;  // weight rows per slice, expert rows per pass
constexpr int kDecMaxExperts = 1024;
constexpr int kDecDeep = 4;   // 32-k steps of loads in flight per wave

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8_t*>(p);
}

// The work of one workgroup: offsets and a_inv may point to global memory or
// to LDS (the fused kernel below computes them in LDS).
template <int D>
__device__ __forceinline__ void decode_units(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, const int32_t* offsets,
    int E_l, int K, int N_out, int gated, uint16_t* __restrict__ C, int act, float clamp,
    int batch_m, const int32_t* a_inv, int a_k) {
  __shared__ f32x4_t red[2][kDecWaves][kWave];
  __shared__ int32_t s_exp[kDecMaxExperts];   // experts with rows, in order
  __shared__ int32_t s_row0[kDecMaxExperts];  // their first row
  __shared__ int32_t s_rows[kDecMaxExperts];  // their row count
  __shared__ int32_t s_n;
  const int w = threadIdx.x / kWave;
  const int lane = lane_id();
  const int j = lane & 15;       // weight row in the slice (MFMA column)
  const int kq = lane >> 4;      // 8-element k group of the 32-k step
  const int N_total = gated ? 2 * N_out : N_out;
  const int slices = gated ? N_out / 8 : N_out / kDecRows;
  const int kw = K / kDecWaves;  // this wave's k-range: [w * kw, (w + 1) * kw)
  const int nsteps = kw / 32;    // >= D
  const int kind = act_kind(act, clamp);
  const float cl = act_limit(clamp);

  // The experts that have rows, compacted in order by wave 0 (every
  // workgroup builds the same list), so the work items are only theirs.
  if (w == 0) {
    int n = 0;
    for (int e0 = 0; e0 < E_l; e0 += kWave) {
      const int e = e0 + lane;
      int row0 = 0, rows = 0;
      if (e < E_l) {
        if (batch_m > 0) {
          row0 = e * batch_m;
          rows = min(offsets[e], batch_m);
        } else {
          row0 = offsets[e];
          rows = offsets[e + 1] - row0;
        }
      }
      const uint64_t has = __ballot(rows > 0);
      if (rows > 0) {
        const int at = n + __popcll(has & ((1ull << lane) - 1ull));
        s_exp[at] = e;
        s_row0[at] = row0;
        s_rows[at] = rows;
      }
      n += __popcll(has);
    }
    if (lane == 0) s_n = n;
  }
  __syncthreads();
  const int64_t items = static_cast<int64_t>(s_n) * slices;

  // Work units: (item, pass of 16 expert rows), items blockIdx.x, +grid, ...
  int64_t it = blockIdx.x;
  if (it >= items) return;  // the whole workgroup
  int rg = 0, s = 0, row0 = 0, rows = 0;
  const uint16_t* wp = W;
  const uint16_t* ap = A;
  // pointers of unit (it_, rg_): weight row of this lane's MFMA column and
  // activation row of its MFMA row (past the expert's count the last row
  // repeats; its products land only in output rows that are not stored)
  auto unit = [&](int64_t it_, int rg_, int& s_, int& row0_, int& rows_, const uint16_t*& wp_,
                  const uint16_t*& ap_) {
    const int xi = static_cast<int>(it_ / slices);
    s_ = static_cast<int>(it_ - static_cast<int64_t>(xi) * slices);
    const int e = s_exp[xi];
    row0_ = s_row0[xi];
    rows_ = s_rows[xi];
    const int wrow =
        gated ? (j < 8 ? 8 * s_ + j : N_out + 8 * s_ + (j - 8)) : kDecRows * s_ + j;
    wp_ = W + (static_cast<int64_t>(e) * N_total + wrow) * K + w * kw + kq * 8;
    const int64_t pr = row0_ + min(rg_ + j, rows_ - 1);
    const int64_t src = a_inv ? a_inv[pr] / a_k : pr;
    ap_ = A + src * K + w * kw + kq * 8;
  };
  unit(it, rg, s, row0, rows, wp, ap);

  // (the weight loads go out first: the activation pointer waits on the
  // inverse-map load)
  bf16x8_t bq[D], aq[D];
#pragma unroll
  for (int d = 0; d < D; ++d) bq[d] = load_bf16x8(wp + d * 32);
#pragma unroll
  for (int d = 0; d < D; ++d) aq[d] = load_bf16x8(ap + d * 32);
  int buf = 0;
  while (true) {
    // the next unit, resolved now so that its inverse-map load lands while
    // this unit streams
    int64_t it2 = it;
    int rg2 = rg + kDecRows;
    if (rg2 >= rows) {
      it2 = it + gridDim.x;
      rg2 = 0;
    }
    const bool more = it2 < items;
    int s2 = s, row02 = row0, rows2 = rows;
    const uint16_t* wp2 = wp;
    const uint16_t* ap2 = ap;
    if (more) unit(it2, rg2, s2, row02, rows2, wp2, ap2);

    f32x4_t acc = {};
    // consume D steps, load the D after them (nsteps is a multiple of D)
    for (int st = 0; st + D < nsteps; st += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[d], bq[d], acc, 0, 0, 0);
        bq[d] = load_bf16x8(wp + (st + D + d) * 32);
        aq[d] = load_bf16x8(ap + (st + D + d) * 32);
      }
    }
    // the next unit's first D steps go out while this one's last D are used
    // and its sums are reduced and stored
#pragma unroll
    for (int d = 0; d < D; ++d) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[d], bq[d], acc, 0, 0, 0);
      if (more) {
        bq[d] = load_bf16x8(wp2 + d * 32);
        aq[d] = load_bf16x8(ap2 + d * 32);
      }
    }

    // the waves' sums over their k-ranges (two buffers: the next unit writes
    // the other one, and this one is rewritten only after the next barrier,
    // which wave 0 reaches once it has read it)
    red[buf][w][lane] = acc;
    __syncthreads();
    if (w == 0) {
      f32x4_t sum = red[buf][0][lane];
#pragma unroll
      for (int ww = 1; ww < kDecWaves; ++ww) sum += red[buf][ww][lane];
      // lane holds rows 4 * kq + i (i < 4) of column j
      if (gated) {
        f32x4_t up;
#pragma unroll
        for (int i = 0; i < 4; ++i) up[i] = __shfl(sum[i], lane + 8, kWave);
        if (j < 8) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = rg + 4 * kq + i;
            if (r >= rows) break;
            float v;
            if (kind == 0) v = gated_act_k<0>(sum[i], up[i], cl);
            else if (kind == 1) v = gated_act_k<1>(sum[i], up[i], cl);
            else v = gated_act_k<2>(sum[i], up[i], cl);
            C[static_cast<int64_t>(row0 + r) * N_out + 8 * s + j] = f32_to_bf16(v);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rg + 4 * kq + i;
          if (r >= rows) break;
          C[static_cast<int64_t>(row0 + r) * N_out + kDecRows * s + j] = f32_to_bf16(sum[i]);
        }
      }
    }
    if (!more) break;
    it = it2;
    rg = rg2;
    s = s2;
    row0 = row02;
    rows = rows2;
    wp = wp2;
    ap = ap2;
    buf ^= 1;
  }
}

template <int D>
__global__ __launch_bounds__(kDecThreads, 4) void decode_gemm_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
    const int32_t* __restrict__ offsets, int E_l, int K, int N_out, int gated,
    uint16_t* __restrict__ C, int act, float clamp, int batch_m, const int32_t* __restrict__ a_inv,
    int a_k) {
  decode_units<D>(A, W, offsets, E_l, K, N_out, gated, C, act, clamp, batch_m, a_inv, a_k);
}

// Router, permute map and GEMM1 of a batch of at most 64 routes in one
// launch.  Every workgroup routes the tokens itself (wave t takes token t;
// the same code on the same logits gives the same picks everywhere), sorts
// the routes by local expert in LDS with one wave (wave_match ranks, counts,
// a scan over the experts) and then runs its GEMM1 work units on the token
// rows through that LDS inverse map; workgroup 0 alone writes the ids,
// weights, map, offsets and inverse map that GEMM2 and finalize read.  The
// results equal those of the router, permute and gathered GEMM1 calls.
template <int EPL, int D>
__global__ __launch_bounds__(kDecThreads, 4) void decode_route_gemm1_kernel(
    const float* __restrict__ logits, int T, int E, int k, int score_fn, int renormalize,
    float rsf, int32_t* __restrict__ ids, float* __restrict__ wts, uint16_t* __restrict__ w_bf16,
    const int32_t* __restrict__ emap, int E_l, int32_t* __restrict__ map,
    int32_t* __restrict__ offsets, int32_t* __restrict__ inv, int64_t R_pad,
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, int K, int N_out,
    uint16_t* __restrict__ C, int act, float clamp) {
  __shared__ int32_t s_loc[kWave];                 // local expert of each route
  __shared__ int32_t s_cnt[kDecMaxExperts];        // routes per local expert
  __shared__ int32_t s_off[kDecMaxExperts + 1];    // their first rows
  __shared__ int32_t s_inv[kWave];                 // route of each row
  const bool lead = blockIdx.x == 0;
  const int w = threadIdx.x / kWave;
  const int lane = lane_id();
  const int R = T * k;  // <= 64
  for (int e = threadIdx.x; e < E_l; e += kDecThreads) s_cnt[e] = 0;
  if (w < T) {
    int em[EPL];
    load_local_map<EPL>(emap, E, E_l, em);
    const int id = route_token<EPL>(logits, w, E, k, score_fn, renormalize, rsf, ids, wts,
                                    w_bf16, lead);
    const int l = local_of_pick<EPL>(em, id, E);
    if (lane < k) s_loc[w * k + lane] = l;
  }
  __syncthreads();
  if (w == 0) {
    // rank of each route among equal experts (ascending route index), the
    // counts, then offsets by a scan over the experts
    const bool valid = lane < R;
    const int L = valid ? s_loc[lane] : -1;
    const uint64_t lt = (1ull << lane) - 1ull;
    const uint64_t peers = wave_match(static_cast<uint32_t>(L + 1), valid, 32 - __clz(E_l));
    if (valid && L >= 0 && (peers & lt) == 0ull) s_cnt[L] = __popcll(peers);
    int run = 0;
    for (int e0 = 0; e0 < E_l; e0 += kWave) {
      const int e = e0 + lane;
      const int c = e < E_l ? s_cnt[e] : 0;
      const int incl = wave_inclusive_sum(c);
      if (e < E_l) {
        s_off[e] = run + incl - c;
        if (lead) offsets[e] = run + incl - c;
      }
      run += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) {
      s_off[E_l] = run;
      if (lead) offsets[E_l] = run;
    }
    if (valid) {
      const int slot = L >= 0 ? s_off[L] + __popcll(peers & lt) : -1;
      if (L >= 0) s_inv[slot] = lane;
      if (lead) {
        map[lane] = slot;
        if (L >= 0 && inv) inv[slot] = lane;
      }
    }
    if (lead && inv)
      for (int64_t r = run + lane; r < R_pad; r += kWave) inv[r] = -1;
  }
  __syncthreads();
  decode_units<D>(X, W, s_off, E_l, K, N_out, 1, C, act, clamp, 0, s_inv, k);
}

// FP8 E4M3 rows with one fp32 scale per row and FP8 E4M3 weights with one
// fp32 scale per weight row, for the same decode batches: decode_units' work
// units, eight waves splitting the k-range.  A 64-k step is 16 bytes a lane,
// four lanes covering a row's 64-byte run as for bf16, with four, two or one
// steps in flight per wave (the deepest that divides the wave's steps: two
// for k = 7168, four for 2048).  Against the split tiles on decode batches
// of DeepSeek-V3 widths: 5-13 % faster (four waves: 3-8 %).  It feeds the 16 x 16 x 128 MFMA (E4M3 for both
// operands, unit block scales) in the first 16 of the 32 operand bytes a
// lane holds, the other 16 zero: both operands place each k in the same
// slot, so the step's products are each summed once whatever the slot
// order.  The row and weight scales multiply the sums after the k-loop.
typedef int i32x8_t __attribute__((ext_vector_type(8)));
constexpr int kF8Waves = 8;
constexpr int kF8Threads = kF8Waves * kWave;

__device__ __forceinline__ uint4 load_u8x16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ f32x4_t mfma_fp8_step(uint4 a, uint4 b, f32x4_t acc) {
  const i32x8_t av = {static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z),
                      static_cast<int>(a.w), 0, 0, 0, 0};
  const i32x8_t bv = {static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z),
                      static_cast<int>(b.w), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
}

template <int D>
__device__ __forceinline__ void decode_units_fp8(
    const uint8_t* __restrict__ A, const float* __restrict__ a_scales,
    const uint8_t* __restrict__ W, const float* __restrict__ w_scales,
    const int32_t* __restrict__ offsets, int E_l, int K, int N_out, int gated,
    uint16_t* __restrict__ C, int act, float clamp, int batch_m, const int32_t* a_inv,
    int a_k) {
  __shared__ f32x4_t red[2][kF8Waves][kWave];
  __shared__ int32_t s_exp[kDecMaxExperts];   // experts with rows, in order
  __shared__ int32_t s_row0[kDecMaxExperts];  // their first row
  __shared__ int32_t s_rows[kDecMaxExperts];  // their row count
  __shared__ int32_t s_n;
  const int w = threadIdx.x / kWave;
  const int lane = lane_id();
  const int j = lane & 15;       // weight row in the slice (MFMA column)
  const int kq = lane >> 4;      // 16-byte k group of the 64-k step
  const int N_total = gated ? 2 * N_out : N_out;
  const int slices = gated ? N_out / 8 : N_out / kDecRows;
  const int kw = K / kF8Waves;   // this wave's k-range: [w * kw, (w + 1) * kw)
  const int nsteps = kw / 64;    // >= D
  const int kind = act_kind(act, clamp);
  const float cl = act_limit(clamp);

  // the experts that have rows, compacted in order by wave 0
  if (w == 0) {
    int n = 0;
    for (int e0 = 0; e0 < E_l; e0 += kWave) {
      const int e = e0 + lane;
      int row0 = 0, rows = 0;
      if (e < E_l) {
        if (batch_m > 0) {
          row0 = e * batch_m;
          rows = min(offsets[e], batch_m);
        } else {
          row0 = offsets[e];
          rows = offsets[e + 1] - row0;
        }
      }
      const uint64_t has = __ballot(rows > 0);
      if (rows > 0) {
        const int at = n + __popcll(has & ((1ull << lane) - 1ull));
        s_exp[at] = e;
        s_row0[at] = row0;
        s_rows[at] = rows;
      }
      n += __popcll(has);
    }
    if (lane == 0) s_n = n;
  }
  __syncthreads();
  const int64_t items = static_cast<int64_t>(s_n) * slices;

  int64_t it = blockIdx.x;
  if (it >= items) return;  // the whole workgroup
  int rg = 0, s = 0, row0 = 0, rows = 0;
  const uint8_t* wp = W;
  const uint8_t* ap = A;
  float wsc = 0.0f, asc = 0.0f;
  // pointers and scales of unit (it_, rg_): this lane's MFMA column (weight
  // row) and MFMA row (activation row; past the expert's count the last row
  // repeats, its products landing only in output rows that are not stored)
  auto unit = [&](int64_t it_, int rg_, int& s_, int& row0_, int& rows_, const uint8_t*& wp_,
                  const uint8_t*& ap_, float& wsc_, float& asc_) {
    const int xi = static_cast<int>(it_ / slices);
    s_ = static_cast<int>(it_ - static_cast<int64_t>(xi) * slices);
    const int e = s_exp[xi];
    row0_ = s_row0[xi];
    rows_ = s_rows[xi];
    const int wrow =
        gated ? (j < 8 ? 8 * s_ + j : N_out + 8 * s_ + (j - 8)) : kDecRows * s_ + j;
    const int64_t widx = static_cast<int64_t>(e) * N_total + wrow;
    wp_ = W + widx * K + w * kw + kq * 16;
    wsc_ = w_scales[widx];
    const int64_t pr = row0_ + min(rg_ + j, rows_ - 1);
    const int64_t src = a_inv ? a_inv[pr] / a_k : pr;
    ap_ = A + src * K + w * kw + kq * 16;
    asc_ = a_scales[src];
  };
  unit(it, rg, s, row0, rows, wp, ap, wsc, asc);

  uint4 bq[D], aq[D];
#pragma unroll
  for (int d = 0; d < D; ++d) bq[d] = load_u8x16(wp + d * 64);
#pragma unroll
  for (int d = 0; d < D; ++d) aq[d] = load_u8x16(ap + d * 64);
  int buf = 0;
  while (true) {
    int64_t it2 = it;
    int rg2 = rg + kDecRows;
    if (rg2 >= rows) {
      it2 = it + gridDim.x;
      rg2 = 0;
    }
    const bool more = it2 < items;
    int s2 = s, row02 = row0, rows2 = rows;
    const uint8_t* wp2 = wp;
    const uint8_t* ap2 = ap;
    float wsc2 = wsc, asc2 = asc;
    if (more) unit(it2, rg2, s2, row02, rows2, wp2, ap2, wsc2, asc2);

    f32x4_t acc = {};
    for (int st = 0; st + D < nsteps; st += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        acc = mfma_fp8_step(aq[d], bq[d], acc);
        bq[d] = load_u8x16(wp + (st + D + d) * 64);
        aq[d] = load_u8x16(ap + (st + D + d) * 64);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      acc = mfma_fp8_step(aq[d], bq[d], acc);
      if (more) {
        bq[d] = load_u8x16(wp2 + d * 64);
        aq[d] = load_u8x16(ap2 + d * 64);
      }
    }

    red[buf][w][lane] = acc;
    __syncthreads();
    if (w == 0) {
      f32x4_t sum = red[buf][0][lane];
#pragma unroll
      for (int ww = 1; ww < kF8Waves; ++ww) sum += red[buf][ww][lane];
      // lane holds rows 4 * kq + i of column j; the row scale of row r sits
      // in lane r (whose MFMA row it is), the weight scale in this lane
#pragma unroll
      for (int i = 0; i < 4; ++i) sum[i] *= __shfl(asc, 4 * kq + i, kWave) * wsc;
      if (gated) {
        f32x4_t up;
#pragma unroll
        for (int i = 0; i < 4; ++i) up[i] = __shfl(sum[i], lane + 8, kWave);
        if (j < 8) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = rg + 4 * kq + i;
            if (r >= rows) break;
            float v;
            if (kind == 0) v = gated_act_k<0>(sum[i], up[i], cl);
            else if (kind == 1) v = gated_act_k<1>(sum[i], up[i], cl);
            else v = gated_act_k<2>(sum[i], up[i], cl);
            C[static_cast<int64_t>(row0 + r) * N_out + 8 * s + j] = f32_to_bf16(v);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rg + 4 * kq + i;
          if (r >= rows) break;
          C[static_cast<int64_t>(row0 + r) * N_out + kDecRows * s + j] = f32_to_bf16(sum[i]);
        }
      }
    }
    if (!more) break;
    it = it2;
    rg = rg2;
    s = s2;
    row0 = row02;
    rows = rows2;
    wp = wp2;
    ap = ap2;
    wsc = wsc2;
    asc = asc2;
    buf ^= 1;
  }
}

template <int D>
__global__ __launch_bounds__(kF8Threads) void decode_gemm_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ a_scales,
    const uint8_t* __restrict__ W, const float* __restrict__ w_scales,
    const int32_t* __restrict__ offsets, int E_l, int K, int N_out, int gated,
    uint16_t* __restrict__ C, int act, float clamp, int batch_m, const int32_t* __restrict__ a_inv,
    int a_k) {
  decode_units_fp8<D>(A, a_scales, W, w_scales, offsets, E_l, K, N_out, gated, C, act, clamp,
                      batch_m, a_inv, a_k);
}

}  // namespace

bool decode_gemm_fits(const GemmArgs& g) {
  return g.a_scales == nullptr && g.w_scales == nullptr && g.K >= kDecWaves * 32 &&
         g.K % (kDecWaves * 32) == 0 &&
         (g.gated ? g.N_out % 8 == 0 : g.N_out % kDecRows == 0) && g.E_l > 0 &&
         g.E_l <= kDecMaxExperts;
}

hipError_t launch_decode_gemm(const GemmArgs& g, hipStream_t s) {
  const int slices = g.gated ? g.N_out / 8 : g.N_out / kDecRows;
  const int64_t items = static_cast<int64_t>(g.E_l) * slices;  // at most
  // four 32-k steps in flight per wave when each wave's k-range is a
  // multiple of four steps (two workgroups fit a compute unit)
  const bool deep = (g.K / kDecWaves / 32) % kDecDeep == 0;
  auto kern = deep ? decode_gemm_kernel<kDecDeep> : decode_gemm_kernel<1>;
  // one resident wave of workgroups; work item i (slice i mod slices of the
  // (i / slices)-th expert with rows) goes to workgroup i mod grid
  static int occ[2] = {0, 0};
  int& o = occ[deep ? 1 : 0];
  if (o == 0) {
    int n = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &n, reinterpret_cast<const void*>(kern), kDecThreads, 0);
    if (e != hipSuccess) return e;
    o = n > 0 ? n : 1;
  }
  int64_t grid = static_cast<int64_t>(device_cu_count()) * o;
  if (grid > items) grid = items;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kDecThreads), 0, s,
                     static_cast<const uint16_t*>(g.a), static_cast<const uint16_t*>(g.w),
                     g.offsets, g.E_l, g.K, g.N_out, g.gated, static_cast<uint16_t*>(g.c), g.act,
                     g.clamp, g.batch_m, g.a_inv, g.a_k);
  return hipGetLastError();
}

bool decode_gemm_fp8_fits(const GemmArgs& g) {
  return g.a_scales != nullptr && g.w_scales != nullptr && !g.w_mxfp4 && g.a_terms == 1 &&
         g.a_ld == 0 && g.K >= kF8Waves * 64 && g.K % (kF8Waves * 64) == 0 &&
         (g.gated ? g.N_out % 8 == 0 : g.N_out % kDecRows == 0) && g.E_l > 0 &&
         g.E_l <= kDecMaxExperts;
}

hipError_t launch_decode_gemm_fp8(const GemmArgs& g, hipStream_t s) {
  const int slices = g.gated ? g.N_out / 8 : g.N_out / kDecRows;
  const int64_t items = static_cast<int64_t>(g.E_l) * slices;  // at most
  // 64-k steps in flight per wave: four, two or one, the deepest that
  // divides the wave's k-range
  const int ns = g.K / kF8Waves / 64;
  const int dsel = ns % 4 == 0 ? 2 : ns % 2 == 0 ? 1 : 0;
  auto kern = dsel == 2 ? decode_gemm_fp8_kernel<4>
            : dsel == 1 ? decode_gemm_fp8_kernel<2> : decode_gemm_fp8_kernel<1>;
  static int occ[3] = {0, 0, 0};
  int& o = occ[dsel];
  if (o == 0) {
    int n = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &n, reinterpret_cast<const void*>(kern), kF8Threads, 0);
    if (e != hipSuccess) return e;
    o = n > 0 ? n : 1;
  }
  int64_t grid = static_cast<int64_t>(device_cu_count()) * o;
  if (grid > items) grid = items;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kF8Threads), 0, s,
                     static_cast<const uint8_t*>(g.a), g.a_scales,
                     static_cast<const uint8_t*>(g.w), static_cast<const float*>(g.w_scales),
                     g.offsets, g.E_l, g.K, g.N_out, g.gated, static_cast<uint16_t*>(g.c), g.act,
                     g.clamp, g.batch_m, g.a_inv, g.a_k);
  return hipGetLastError();
}

namespace {
template <int EPL>
hipError_t launch_fused_epl(const float* logits, int T, int E, int k, int score_fn, int renorm,
                            float rsf, int32_t* ids, float* wts, uint16_t* w_bf16,
                            const int32_t* emap, int E_l, int32_t* map, int32_t* offsets,
                            int32_t* inv, int64_t R_pad, const GemmArgs& g, hipStream_t s) {
  const bool deep = (g.K / kDecWaves / 32) % kDecDeep == 0;
  auto kern = deep ? decode_route_gemm1_kernel<EPL, kDecDeep> : decode_route_gemm1_kernel<EPL, 1>;
  static int occ[2] = {0, 0};
  int& o = occ[deep ? 1 : 0];
  if (o == 0) {
    int n = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &n, reinterpret_cast<const void*>(kern), kDecThreads, 0);
    if (e != hipSuccess) return e;
    o = n > 0 ? n : 1;
  }
  const int slices = g.N_out / 8;
  const int64_t items = static_cast<int64_t>(g.E_l) * slices;  // at most
  int64_t grid = static_cast<int64_t>(device_cu_count()) * o;
  if (grid > items) grid = items;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kDecThreads), 0, s, logits, T,
                     E, k, score_fn, renorm, rsf, ids, wts, w_bf16, emap, E_l, map, offsets, inv,
                     R_pad, static_cast<const uint16_t*>(g.a), static_cast<const uint16_t*>(g.w),
                     g.K, g.N_out, static_cast<uint16_t*>(g.c), g.act, g.clamp);
  return hipGetLastError();
}
}  // namespace

bool decode_route_gemm1_fits(const GemmArgs& g, int64_t T, int E, int k) {
  return g.gated && decode_gemm_fits(g) && g.batch_m == 0 && T >= 1 && T * k <= kWave &&
         T <= kDecWaves && E <= 1024;
}

hipError_t launch_decode_route_gemm1(const float* logits, int64_t T, int E, int k, int score_fn,
                                     int renormalize, float rsf, int32_t* ids, float* wts,
                                     uint16_t* w_bf16, const int32_t* emap, int32_t* map,
                                     int32_t* offsets, int32_t* inv, int64_t R_pad,
                                     const GemmArgs& g, hipStream_t s) {
  const int epl = (E + kWave - 1) / kWave;
  const int Ti = static_cast<int>(T);
#define MOE_FUSED(N)                                                                          \
  return launch_fused_epl<N>(logits, Ti, E, k, score_fn, renormalize, rsf, ids, wts, w_bf16, \
                             emap, g.E_l, map, offsets, inv, R_pad, g, s)
  if (epl <= 1) MOE_FUSED(1);
  if (epl <= 2) MOE_FUSED(2);
  if (epl <= 4) MOE_FUSED(4);
  if (epl <= 8) MOE_FUSED(8);
  MOE_FUSED(16);
#undef MOE_FUSED
}

}  // namespace moe
