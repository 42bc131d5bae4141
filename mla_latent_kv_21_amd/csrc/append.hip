// mla_cache_append: c = RMSNorm(x · W_DKV) * gamma, k_r = RoPE(x · W_KR, pos), written as one
// [c || k_r] row into the paged latent cache (Smallem article 13, "L'idée : garder un résumé",
// "L'obstacle : RoPE" and the cache extension in "Le code").
//
// Two kernels: a split-K projection of x against [W_DKV | W_KR] into fp32 partial sums (the
// projection is bound by reading the 2*C*(d_c+d_r)-byte weights, so it is spread over many
// workgroups even for a handful of tokens), then one workgroup per token that sums the
// partials in a fixed order, normalises, rotates and stores the row at its slot.
#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kTokTile = 16;   // tokens per projection workgroup
constexpr int kColTile = 64;   // output columns per projection workgroup
constexpr int kKStage = 64;    // k values staged in LDS per step
constexpr int kKChunk = 512;   // C values reduced by one partial sum
constexpr int kMaxTok = 2048;  // tokens per pass of the two kernels

template <typename T>
__global__ __launch_bounds__(256) void append_project(const T* __restrict__ x,
                                                      const T* __restrict__ w_dkv,
                                                      const T* __restrict__ w_kr, int n_tok,
                                                      int C, int d_c, int d_r, int k_chunk,
                                                      float* __restrict__ y_part) {
  __shared__ float xs[kTokTile][kKStage + 1];
  const int ncols = d_c + d_r;
  const int col = blockIdx.x * kColTile + (threadIdx.x & 63);
  const int tr = threadIdx.x >> 6;  // 0..3: token lane
  const int ks = blockIdx.y;
  const int n0 = blockIdx.z * kTokTile;
  const int k0 = ks * k_chunk, k1 = min(C, k0 + k_chunk);
  const T* wcol = nullptr;
  int wstride = 0, wc = 0;
  if (col < d_c) {
    wcol = w_dkv; wstride = d_c; wc = col;
  } else if (col < ncols) {
    wcol = w_kr; wstride = d_r; wc = col - d_c;
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int kk = k0; kk < k1; kk += kKStage) {
    for (int e = threadIdx.x; e < kTokTile * kKStage; e += 256) {
      const int r = e / kKStage, k = e % kKStage;
      const int n = n0 + r, kg = kk + k;
      xs[r][k] = (n < n_tok && kg < k1) ? ld(x, static_cast<int64_t>(n) * C + kg) : 0.f;
    }
    __syncthreads();
    if (wcol != nullptr) {
      const int kn = min(kKStage, k1 - kk);
      for (int k = 0; k < kn; ++k) {
        const float w = ld(wcol, static_cast<int64_t>(kk + k) * wstride + wc);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += xs[tr + 4 * r][k] * w;
      }
    }
    __syncthreads();
  }
  if (col < ncols) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = n0 + tr + 4 * r;
      if (n < n_tok) y_part[(static_cast<int64_t>(ks) * n_tok + n) * ncols + col] = acc[r];
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void append_finalize(
    const float* __restrict__ y_part, int n_ksplit, int n_tok, const T* __restrict__ gamma,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ table, int batch, int max_blocks, int num_blocks, int bs,
    int d_c, int d_r, float eps, float base, T* __restrict__ cache) {
  extern __shared__ float ys[];  // [d_c + d_r]
  __shared__ float red[16];
  const int n = blockIdx.x;
  const int ncols = d_c + d_r;
  float ss = 0.f;
  for (int c = threadIdx.x; c < ncols; c += blockDim.x) {
    float y = 0.f;
    for (int k = 0; k < n_ksplit; ++k) y += y_part[(static_cast<int64_t>(k) * n_tok + n) * ncols + c];
    ys[c] = y;
    if (c < d_c) ss += y * y;
  }
  ss = block_sum(ss, red);  // also orders the ys writes before the reads below
  const int b = seq_idx[n], p = pos[n];
  if (b < 0 || b >= batch) return;
  const int64_t slot = cache_slot(table, max_blocks, bs, num_blocks, b, p);
  if (slot < 0) return;
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(d_c) + eps);
  T* row = cache + slot * ncols;
  for (int c = threadIdx.x; c < d_c; c += blockDim.x) st(row, c, ys[c] * inv * ld(gamma, c));
  for (int j = threadIdx.x; j < d_r / 2; j += blockDim.x) {
    float cs, sn;
    rope_cos_sin(p, j, d_r, base, &cs, &sn);
    const float a = ys[d_c + 2 * j], q = ys[d_c + 2 * j + 1];
    st(row, d_c + 2 * j, a * cs - q * sn);
    st(row, d_c + 2 * j + 1, a * sn + q * cs);
  }
}

}  // namespace

AppendPlan append_plan(const mla_dims& d, int n_tok) {
  // Fixed 512-wide ranges of C per partial sum, added in a fixed order: a row's result does
  // not depend on how many tokens are appended with it. Tokens go through in chunks of at
  // most kMaxTok, which bounds the workspace.
  AppendPlan p;
  const int ncols = d.d_c + d.d_r;
  const int n = n_tok < kMaxTok ? n_tok : kMaxTok;
  p.col_blocks = cdiv(ncols, kColTile);
  p.tok_tiles = cdiv(n > 0 ? n : 1, kTokTile);
  p.k_chunk = kKChunk;
  p.n_ksplit = cdiv(d.d_model, p.k_chunk);
  return p;
}

hipError_t launch_append(const mla_dims& d, int n_tok, const void* x, const int32_t* seq_idx,
                         const int32_t* pos, const void* w_dkv, const void* gamma,
                         const void* w_kr, const int32_t* table, int batch, int max_blocks,
                         int num_blocks, void* cache, void* ws, hipStream_t s) {
  float* y_part = static_cast<float*>(ws);
  const size_t lds = static_cast<size_t>(d.d_c + d.d_r) * sizeof(float);
  const size_t elt = d.dtype == MLA_BF16 ? 2 : 4;
  for (int t0 = 0; t0 < n_tok; t0 += kMaxTok) {
    const int n = n_tok - t0 < kMaxTok ? n_tok - t0 : kMaxTok;
    const AppendPlan p = append_plan(d, n);
    const dim3 g1(p.col_blocks, p.n_ksplit, p.tok_tiles);
    const void* xc = static_cast<const char*>(x) + static_cast<size_t>(t0) * d.d_model * elt;
    if (d.dtype == MLA_BF16) {
      hipLaunchKernelGGL(append_project<bf16>, g1, dim3(256), 0, s, static_cast<const bf16*>(xc),
                         static_cast<const bf16*>(w_dkv), static_cast<const bf16*>(w_kr), n,
                         d.d_model, d.d_c, d.d_r, p.k_chunk, y_part);
      hipLaunchKernelGGL(append_finalize<bf16>, dim3(n), dim3(256), lds, s, y_part, p.n_ksplit,
                         n, static_cast<const bf16*>(gamma), seq_idx + t0, pos + t0, table,
                         batch, max_blocks, num_blocks, d.block_size, d.d_c, d.d_r, d.rms_eps,
                         d.rope_base, static_cast<bf16*>(cache));
    } else {
      hipLaunchKernelGGL(append_project<float>, g1, dim3(256), 0, s,
                         static_cast<const float*>(xc), static_cast<const float*>(w_dkv),
                         static_cast<const float*>(w_kr), n, d.d_model, d.d_c, d.d_r, p.k_chunk,
                         y_part);
      hipLaunchKernelGGL(append_finalize<float>, dim3(n), dim3(256), lds, s, y_part, p.n_ksplit,
                         n, static_cast<const float*>(gamma), seq_idx + t0, pos + t0, table,
                         batch, max_blocks, num_blocks, d.block_size, d.d_c, d.d_r, d.rms_eps,
                         d.rope_base, static_cast<float*>(cache));
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mla
