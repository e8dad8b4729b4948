// The stable counting sort behind Permute (see permute.hip), shared by the
// permute kernel (routes read from the topk ids, one or more workgroups) and
// the merged route-and-permute kernel of small batches (routes kept in LDS by
// the router, one workgroup).
#pragma once

#include "moe_common.h"

namespace moe {
namespace {

constexpr int kPermuteThreads = 1024;
constexpr int kPermuteWaves = kPermuteThreads / kWave;

constexpr int kChunk = 16;  // walk steps whose routes a wave loads at once

// Local expert of route x: expert_map[ids[x]] (ids[x] without a map), -1 when
// not local or when the id lies outside [0, E).
__device__ __forceinline__ int local_of(int id, const int32_t* __restrict__ emap, int E,
                                        int E_l) {
  const int l = (id >= 0 && id < E) ? (emap ? emap[id] : id) : -1;
  return (l >= 0 && l < E_l) ? l : -1;
}

// Routes read from the topk ids in global memory.  load() gives the local
// expert (or -1) of route base + c * 64 + lane for the kChunk steps of a
// chunk; routes at or past `end` read nothing.  The id loads are issued back
// to back, then the expert-map loads, so their latencies overlap.
struct GlobalRoutes {
  const int32_t* __restrict__ ids;
  const int32_t* __restrict__ emap;
  int E, E_l;
  __device__ __forceinline__ void load(int64_t base, int64_t end, int (&L)[kChunk]) const {
    const int lane = lane_id();
    int id[kChunk];
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const int64_t x = base + c * kWave + lane;
      id[c] = x < end ? ids[x] : -1;
    }
#pragma unroll
    for (int c = 0; c < kChunk; ++c) L[c] = local_of(id[c], emap, E, E_l);
  }
};

// Routes whose local experts are already in LDS (one int per route).
struct LdsRoutes {
  const int32_t* L;
  __device__ __forceinline__ void load(int64_t base, int64_t end, int (&Lc)[kChunk]) const {
    const int lane = lane_id();
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const int64_t x = base + c * kWave + lane;
      Lc[c] = x < end ? L[x] : -1;
    }
  }
};

// LDS bytes of the sort: per-wave histograms, the per-expert totals and
// counts before this workgroup's range, and the block-scan scratch.
__host__ __device__ constexpr size_t sort_lds_bytes(int E_l) {
  return sizeof(int32_t) * (static_cast<size_t>(kPermuteWaves + 2) * E_l + 16);
}

// Workgroups of the sort for R routes: one per 1024 routes (one walk step
// per wave), at most 256.
__host__ __device__ constexpr int sort_blocks(int64_t R) {
  return R <= kPermuteThreads ? 1
         : static_cast<int>((R + kPermuteThreads - 1) / kPermuteThreads < 256
                                ? (R + kPermuteThreads - 1) / kPermuteThreads
                                : 256);
}

// The stable counting sort of the R routes of `src` by local expert, run by
// workgroup `blk` of `nblk` (each of kPermuteThreads threads; smem holds
// sort_lds_bytes(E_l)).  Workgroup blk places the routes of its contiguous
// range [beg_b, end_b) of the expanded index:
//   - with several workgroups, each counts all R routes per local expert in
//     LDS (integer LDS adds, whose sums do not depend on their order), both
//     in total and before beg_b, so no workgroup waits for another and no
//     global scratch is needed;
//   - the first row of expert e is then its offset plus the routes to e
//     before beg_b; inside the range, wave w owns a contiguous run of it;
//     per-wave counts, a column scan over the waves and, per step, the rank
//     among equal-keyed lower lanes (wave_match) give each route its row.
// Workgroup 0 writes offsets; map [R] and inv [R_pad] (when given) are
// written by all.
template <class Src>
__device__ __forceinline__ void counting_sort(const Src& src, int64_t R, int E_l,
                                              int32_t* __restrict__ map,
                                              int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ inv, int64_t R_pad,
                                              int batch_m, int32_t* smem, int blk, int nblk) {
  int32_t* hist = smem;                                // [waves][E_l]
  int32_t* tot = smem + kPermuteWaves * E_l;           // [E_l] routes to e
  int32_t* pre = tot + E_l;                            // [E_l] of those before beg_b
  int32_t* scratch = pre + E_l;                        // 16 ints
  __shared__ int32_t s_total;
  const int w = threadIdx.x / kWave;
  const int lane = lane_id();
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  constexpr int64_t kStep = kPermuteWaves * kWave;

  for (int i = threadIdx.x; i < (kPermuteWaves + 2) * E_l; i += kPermuteThreads) smem[i] = 0;
  __syncthreads();

  // this workgroup's range (whole wave steps)
  const int64_t per_blk = ((R + int64_t(nblk) * kWave - 1) / (int64_t(nblk) * kWave)) * kWave;
  const int64_t beg_b = blk * per_blk < R ? blk * per_blk : R;
  const int64_t end_b = beg_b + per_blk < R ? beg_b + per_blk : R;

  const int nbits = 32 - __clz(E_l);  // keys L + 1 lie in [0, E_l]
  // Adds the routes of one step (64 routes from `base`, lane's expert L) to
  // counts row `row`: a few experts (E_l <= 32, where skewed routing would
  // pile many lanes on one LDS word) through one add per distinct expert,
  // found with wave_match; many experts with one LDS atomic per lane.
  auto count_step = [&](int32_t* row, int64_t base, int64_t end, int L) {
    const bool valid = base + lane < end;
    if (E_l <= 32) {
      const uint64_t peers = wave_match(static_cast<uint32_t>(L + 1), valid, nbits);
      if (valid && L >= 0 && (peers & lt_mask) == 0ull) atomicAdd(&row[L], __popcll(peers));
    } else if (valid && L >= 0) {
      atomicAdd(&row[L], 1);
    }
  };

  // Counts over all routes (each wave a contiguous run of [0, R), whole
  // steps, so a step lies wholly before beg_b or not); one workgroup needs
  // none: its own per-wave counts are all of them.
  if (nblk > 1) {
    const int64_t per_wave = ((R + kStep - 1) / kStep) * kWave;
    const int64_t beg = w * per_wave < R ? w * per_wave : R;
    const int64_t end = beg + per_wave < R ? beg + per_wave : R;
    // (the branch on E_l outside the walk keeps each loop body straight-line)
    if (E_l <= 32) {
      for (int64_t cb = beg; cb < end; cb += kChunk * kWave) {
        int Lc[kChunk];
        src.load(cb, end, Lc);
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          const int64_t base = cb + c * kWave;
          if (base >= end) break;  // wave-uniform
          count_step(tot, base, end, Lc[c]);
          if (base < beg_b) count_step(pre, base, end, Lc[c]);
        }
      }
    } else {
      for (int64_t cb = beg; cb < end; cb += kChunk * kWave) {
        int Lc[kChunk];
        src.load(cb, end, Lc);
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          const int64_t x = cb + c * kWave + lane;
          if (x < end && Lc[c] >= 0) {
            atomicAdd(&tot[Lc[c]], 1);
            if (x < beg_b) atomicAdd(&pre[Lc[c]], 1);
          }
        }
      }
    }
  }

  // Per-wave counts over this workgroup's range.  A run of at most one chunk
  // (the usual case: about 1024 routes per workgroup) keeps its experts in
  // registers for the ranking walk below.
  const int64_t span = end_b - beg_b;
  const int64_t per_wave = ((span + kStep - 1) / kStep) * kWave;
  // waves whose run is not empty (all 16 but for small ranges)
  const int nwa =
      per_wave > 0 ? static_cast<int>(min(static_cast<int64_t>(kPermuteWaves),
                                          (span + per_wave - 1) / per_wave))
                   : 0;
  const int64_t beg = beg_b + (w * per_wave < span ? w * per_wave : span);
  const int64_t end = beg + per_wave < end_b ? beg + per_wave : end_b;
  const bool one_chunk = end - beg <= kChunk * kWave;
  int32_t* my_hist = hist + w * E_l;
  int Lk[kChunk];
  if (one_chunk) src.load(beg, end, Lk);
  auto walk = [&](auto&& step) {
    if (one_chunk) {
#pragma unroll
      for (int c = 0; c < kChunk; ++c) {
        const int64_t base = beg + c * kWave;
        if (base >= end) break;  // wave-uniform
        step(base, Lk[c]);
      }
      return;
    }
    for (int64_t cb = beg; cb < end; cb += kChunk * kWave) {
      int Lc[kChunk];
      src.load(cb, end, Lc);
#pragma unroll
      for (int c = 0; c < kChunk; ++c) {
        const int64_t base = cb + c * kWave;
        if (base >= end) break;  // wave-uniform
        step(base, Lc[c]);
      }
    }
  };
  walk([&](int64_t base, int L) { count_step(my_hist, base, end, L); });
  __syncthreads();

  // Column scan over waves: hist[w][e] becomes the count of routes to e in
  // earlier waves of this range; the per-expert totals go through a block
  // scan; then every row gets the expert's first row for this range.
  const int e = threadIdx.x;  // E_l <= kPermuteThreads
  int cnt_total = 0;
  if (e < E_l) {
    int run = 0;
    for (int ww = 0; ww < nwa; ++ww) {
      const int c = hist[ww * E_l + e];
      hist[ww * E_l + e] = run;
      run += c;
    }
    cnt_total = nblk > 1 ? tot[e] : run;
  }
  int total = 0;
  const int start = block_exclusive_sum(e < E_l ? cnt_total : 0, scratch, &total);
  if (e < E_l) {
    const int base = (batch_m > 0 ? e * batch_m : start) + pre[e];
    if (blk == 0) offsets[e] = batch_m > 0 ? cnt_total : start;
    for (int ww = 0; ww < nwa; ++ww) hist[ww * E_l + e] += base;
  }
  if (threadIdx.x == 0) {
    if (blk == 0 && batch_m == 0) offsets[E_l] = total;
    s_total = total;
  }
  __syncthreads();

  // Ranks, map and inverse map over this workgroup's range.
  walk([&](int64_t base, int L) {
    const int64_t x = base + lane;
    const bool valid = x < end;
    const uint64_t peers = wave_match(static_cast<uint32_t>(L + 1), valid, nbits);
    if (valid) {
      if (L >= 0) {
        const int slot = my_hist[L] + __popcll(peers & lt_mask);
        if (batch_m > 0 && slot - L * batch_m >= batch_m) {
          map[x] = -1;  // past the expert's capacity
        } else {
          map[x] = slot;
          if (inv) inv[slot] = static_cast<int32_t>(x);
        }
      } else {
        map[x] = -1;
      }
    }
    // every lane has read its row of my_hist above before the leader adds
    if (valid && L >= 0 && (peers & lt_mask) == 0ull) my_hist[L] += __popcll(peers);
  });
  if (inv) {
    for (int64_t r = s_total + int64_t(blk) * kPermuteThreads + threadIdx.x; r < R_pad;
         r += int64_t(nblk) * kPermuteThreads)
      inv[r] = -1;
  }
}

}  // namespace
}  // namespace moe
