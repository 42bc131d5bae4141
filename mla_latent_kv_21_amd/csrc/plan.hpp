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
// Every split workgroup computes the same plan from the lengths; slot 0 also stores it in the
// workspace, where the merge reads it.
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

// Sum and max over the thread block (blockDim.x a multiple of 64, at most 1024); `red` holds
// 32 ints of LDS.
__device__ __forceinline__ int64_t plan_block_sum(int64_t v, int* red) {
  long long s = v;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    red[2 * w] = static_cast<int>(s & 0xffffffff);
    red[2 * w + 1] = static_cast<int>(s >> 32);
  }
  __syncthreads();
  int64_t t = 0;
  for (int i = 0; i < nw; ++i)
    t += static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(red[2 * i + 1])) << 32) |
                              static_cast<uint32_t>(red[2 * i]));
  return t;
}

__device__ __forceinline__ int plan_block_max(int v, int* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  int t = red[0];
  for (int i = 1; i < nw; ++i) t = max(t, red[i]);
  return t;
}

// The plan for `rows` = batch * s_q <= kPlanMaxRows query rows, computed by the whole thread
// block into *p (LDS); `red` is 32 ints of LDS scratch.
__device__ inline void make_plan(const int32_t* __restrict__ lens, int batch, int s_q,
                                 int capacity, SplitPlan* p, int* red) {
  const int rows = batch * s_q;
  // row lengths (visible positions) go through p->first as scratch
  int64_t wsum = 0;
  int lmax = 0;
  for (int m = threadIdx.x; m < rows; m += blockDim.x) {
    const int lim = visible_count(lens[m / s_q], s_q, m % s_q, capacity);
    p->first[m] = lim;
    wsum += lim;
    lmax = max(lmax, lim);
  }
  const int64_t W = plan_block_sum(wsum, red);
  lmax = plan_block_max(lmax, red);
  const int64_t a = kSplitAlign;
  auto up = [&](int64_t x) { return (x + a - 1) / a * a; };
  int64_t lo = up(max(max((W + kPlanSlots - 1) / kPlanSlots, static_cast<int64_t>(lmax + kPlanCap - 1) / kPlanCap),
                      static_cast<int64_t>(1)));
  // with chunk >= W / (kPlanSlots - rows), the rows need at most W / chunk + rows <= kPlanSlots
  int64_t hi = max(lo, up((W + (kPlanSlots - rows) - 1) / (kPlanSlots - rows)));
  // smallest chunk in [lo, hi] (multiples of kSplitAlign) whose split count fits: the count
  // never grows with the chunk
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / (2 * a) * a;
    int64_t cnt = 0;
    for (int m = threadIdx.x; m < rows; m += blockDim.x) cnt += (p->first[m] + mid - 1) / mid;
    if (plan_block_sum(cnt, red) <= kPlanSlots)
      hi = mid;
    else
      lo = mid + a;
  }
  const int chunk = static_cast<int>(lo);
  __syncthreads();
  // first[] as the exclusive prefix of the per-row split counts, by wave 0 in 64-row pieces
  if (threadIdx.x < 64) {
    int carry = 0;
    for (int base = 0; base < rows; base += 64) {
      const int m = base + static_cast<int>(threadIdx.x);
      const int n = m < rows ? (p->first[m] + chunk - 1) / chunk : 0;
      int incl = n;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (static_cast<int>(threadIdx.x) >= o) incl += t;
      }
      if (m < rows) p->first[m] = carry + incl - n;
      carry += __shfl(incl, 63, 64);
    }
    if (threadIdx.x == 0) {
      p->first[rows] = carry;
      p->total = carry;
      p->chunk = chunk;
    }
  }
  __syncthreads();
}

}  // namespace mla
