// gqla_expand: rebuild the G key groups and G value groups of every cached position once,
// [c · W_UK[:, 0..G-1] || c · W_UV[:, 0..G-1] || k_r], into the expanded GQA cache (GQLA summary,
// section 2, "Chemin GQA": the latent is expanded once, and decode then runs plain GQA with no
// expansion per step).
//
// A tiled product over 64 positions x 64 output columns per workgroup, latents gathered
// through the block table into LDS; the workgroups of column tile 0 also copy k_r.
#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kRowT = 64, kColT = 64, kKT = 32;

template <typename T>
__global__ __launch_bounds__(256) void expand_kernel(
    const T* __restrict__ latent, int num_blocks, const int32_t* __restrict__ table,
    int max_blocks, const int32_t* __restrict__ lens, const int32_t* __restrict__ start_pos,
    int bs, int d_c, int d_r, int G, int D, int Dv, const T* __restrict__ w_uk,
    const T* __restrict__ w_uv, T* __restrict__ gqa) {
  __shared__ float cs[kRowT][kKT + 1];
  __shared__ float ws[kKT][kColT + 1];
  __shared__ int64_t slots[kRowT];
  const int b = blockIdx.y;
  const int p0 = blockIdx.x * kRowT;
  const int capacity = max_blocks * bs;
  int L = lens[b];
  L = L > capacity ? capacity : L;
  int P0 = start_pos != nullptr ? start_pos[b] : 0;
  P0 = P0 < 0 ? 0 : P0;
  if (p0 + kRowT <= P0 || p0 >= L) return;
  const int row_w = d_c + d_r;
  const int gw = G * D + G * Dv + d_r;
  for (int r = threadIdx.x; r < kRowT; r += blockDim.x) {
    const int p = p0 + r;
    slots[r] = (p >= P0 && p < L) ? cache_slot(table, max_blocks, bs, num_blocks, b, p) : -1;
  }
  __syncthreads();
  const int c0 = blockIdx.z * kColT;
  const int ncol = G * D + G * Dv;
  const int tr = (threadIdx.x >> 4) * 4, tc = (threadIdx.x & 15) * 4;
  float acc[4][4] = {};
  for (int kk = 0; kk < d_c; kk += kKT) {
    for (int e = threadIdx.x; e < kRowT * kKT; e += blockDim.x) {
      const int r = e / kKT, k = e % kKT;
      const int64_t sl = slots[r];
      cs[r][k] = (sl >= 0 && kk + k < d_c) ? ld(latent, sl * row_w + kk + k) : 0.f;
    }
    for (int e = threadIdx.x; e < kKT * kColT; e += blockDim.x) {
      const int k = e / kColT, c = e % kColT;
      const int col = c0 + c, kg = kk + k;
      float w = 0.f;
      if (kg < d_c && col < ncol) {
        w = col < G * D ? ld(w_uk, static_cast<int64_t>(kg) * (G * D) + col)
                        : ld(w_uv, static_cast<int64_t>(kg) * (G * Dv) + (col - G * D));
      }
      ws[k][c] = w;
    }
    __syncthreads();
    for (int k = 0; k < kKT; ++k) {
      float cv[4], wv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) { cv[u] = cs[tr + u][k]; wv[u] = ws[k][tc + u]; }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] += cv[u] * wv[v];
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t sl = slots[tr + u];
    if (sl < 0) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int col = c0 + tc + v;
      if (col < ncol) st(gqa, sl * gw + col, acc[u][v]);
    }
  }
  if (blockIdx.z == 0) {
    for (int e = threadIdx.x; e < kRowT * d_r; e += blockDim.x) {
      const int r = e / d_r, j = e % d_r;
      const int64_t sl = slots[r];
      if (sl >= 0) st(gqa, sl * gw + ncol + j, ld(latent, sl * row_w + d_c + j));
    }
  }
}

}  // namespace

hipError_t launch_expand(const mla_dims& d, int batch, const void* cache, int num_blocks,
                         const int32_t* table, int max_blocks, const int32_t* seq_lens,
                         const int32_t* start_pos, const void* w_uk, const void* w_uv,
                         void* gqa, hipStream_t s) {
  const int ncol = d.n_groups * (d.d_nope + d.d_v);
  const dim3 grid(cdiv(max_blocks * d.block_size, kRowT), batch, cdiv(ncol, kColT));
  if (d.dtype == MLA_BF16) {
    hipLaunchKernelGGL(expand_kernel<bf16>, grid, dim3(256), 0, s, static_cast<const bf16*>(cache),
                       num_blocks, table, max_blocks, seq_lens, start_pos, d.block_size, d.d_c,
                       d.d_r, d.n_groups, d.d_nope, d.d_v, static_cast<const bf16*>(w_uk),
                       static_cast<const bf16*>(w_uv), static_cast<bf16*>(gqa));
  } else {
    hipLaunchKernelGGL(expand_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(cache), num_blocks, table, max_blocks, seq_lens,
                       start_pos, d.block_size, d.d_c, d.d_r, d.n_groups, d.d_nope, d.d_v,
                       static_cast<const float*>(w_uk), static_cast<const float*>(w_uv),
                       static_cast<float*>(gqa));
  }
  return hipGetLastError();
}

}  // namespace mla
