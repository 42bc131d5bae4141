// Length-balanced split plan of the absorbed decode (n_split = 0 on the matrix-core path).
//
// With a uniform split every (sequence, query) row is cut into the same number of chunks, so a
// batch of mixed lengths leaves the short rows' workgroups idle while the long rows' ones run:
// the step takes as long as the longest chunk. The balanced plan cuts every row into chunks of
// one common size instead, chosen on the device from the lengths:
//  * chunk = the smallest multiple of kSplitAlign for which all rows together need at most
//    kPlanSlots splits (one workgroup per CU) and no row needs more than kPlanCap;
//  * row m = b s_q + i takes splits first[m] .. first[m+1]-1; split slot s covers positions
//    [k chunk, min((k+1) chunk, lim_m)) of its row, k = s - first[m];
//  * partials are indexed by slot: row s H + h of the partial rows, flag s of the flags.
// Every split workgroup computes the same plan from the lengths (one wave, no block-wide
// reductions); slot 0 also stores it in the workspace, where the merge reads it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "launch.hpp"

namespace mla {

constexpr int kPlanSlots = 256;    // split workgroups of a balanced plan (one per CU)
constexpr int kPlanMaxRows = 128;  // query rows (batch x s_q) a balanced plan covers
constexpr int kPlanCap = 64;       // most splits of one row
constexpr size_t kPlanBytes = 1024;  // workspace bytes reserved for the plan

struct SplitPlan {
  int chunk;                    // positions per split, a multiple of kSplitAlign
  int total;                    // splits of all rows, <= kPlanSlots
  int first[kPlanMaxRows + 1];  // first slot of row m; first[rows] = total
};
static_assert(sizeof(SplitPlan) <= kPlanBytes, "plan fits its workspace reserve");

// Wave-wide sum and max (64 lanes).
__device__ __forceinline__ int64_t plan_wave_sum(int64_t v) {
  long long s = v;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  return s;
}
__device__ __forceinline__ int plan_wave_sum32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int plan_wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}
// inclusive prefix sum over the wave's lanes
__device__ __forceinline__ int plan_wave_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// The plan for `rows` = batch * s_q <= kPlanMaxRows query rows into *p (LDS), and in row_of[0]
// the row that split slot `slot` belongs to (-1 past the last split), in row_of[1] that row's
// visible length. Wave 0 computes it alone
// (lane l holds rows l and l + 64), with wave-level reductions only; the one barrier at the end
// publishes it to the whole block, which must call this together.
__device__ inline void make_plan(const int32_t* __restrict__ lens, int batch, int s_q,
                                 int capacity, int slot, SplitPlan* p, int* row_of) {
  const int rows = batch * s_q;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int lim[2];
    int64_t wsum = 0;
    int lmax = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int m = lane + 64 * j;
      lim[j] = m < rows ? visible_count(lens[m / s_q], s_q, m % s_q, capacity) : 0;
      wsum += lim[j];
      lmax = max(lmax, lim[j]);
    }
    const int64_t W = plan_wave_sum(wsum);
    lmax = plan_wave_max(lmax);
    const int64_t a = kSplitAlign;
    auto up = [&](int64_t x) { return (x + a - 1) / a * a; };
    int64_t lo = up(max(max((W + kPlanSlots - 1) / kPlanSlots,
                            static_cast<int64_t>(lmax + kPlanCap - 1) / kPlanCap),
                        static_cast<int64_t>(1)));
    // with chunk >= W / (kPlanSlots - rows), the rows need at most W / chunk + rows <= kPlanSlots
    int64_t hi = max(lo, up((W + (kPlanSlots - rows) - 1) / (kPlanSlots - rows)));
    // smallest chunk in [lo, hi] (multiples of kSplitAlign) whose split count fits: the count
    // never grows with the chunk. With rows <= 128, hi is at most the longest row rounded up,
    // so 32-bit unsigned divisions hold every quotient.
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / (2 * a) * a;
      const unsigned um = static_cast<unsigned>(mid);
      const int c = static_cast<int>((static_cast<unsigned>(lim[0]) + um - 1) / um +
                                     (static_cast<unsigned>(lim[1]) + um - 1) / um);
      const int cnt = plan_wave_sum32(c);
      if (cnt <= kPlanSlots)
        hi = mid;
      else
        lo = mid + a;
    }
    const int chunk = static_cast<int>(lo);
    // first[] as the exclusive prefix of the per-row split counts, rows in order
    const unsigned uc = static_cast<unsigned>(chunk);
    const int n0 = static_cast<int>((static_cast<unsigned>(lim[0]) + uc - 1) / uc);
    const int n1 = static_cast<int>((static_cast<unsigned>(lim[1]) + uc - 1) / uc);
    const int i0 = plan_wave_scan(n0, lane);
    const int carry = __shfl(i0, 63, 64);
    const int i1 = plan_wave_scan(n1, lane);
    const int total = carry + __shfl(i1, 63, 64);
    const int f0 = i0 - n0, f1 = carry + i1 - n1;
    if (lane < rows) p->first[lane] = f0;
    if (lane + 64 < rows) p->first[lane + 64] = f1;
    // the row of `slot`: the one whose splits [first, first + n) hold it
    const bool h0 = lane < rows && f0 <= slot && slot < f0 + n0;
    const bool h1 = lane + 64 < rows && f1 <= slot && slot < f1 + n1;
    if (h0) row_of[1] = lim[0];
    if (h1) row_of[1] = lim[1];
    const unsigned long long b0 = __ballot(h0), b1 = __ballot(h1);
    if (lane == 0) {
      p->first[rows] = total;
      p->total = total;
      p->chunk = chunk;
      *row_of = b0 ? __builtin_ctzll(b0) : b1 ? 64 + __builtin_ctzll(b1) : -1;
    }
  }
  __syncthreads();
}

}  // namespace mla
