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
constexpr int kKStage = 256;   // k values staged in LDS per step (one k_chunk)
constexpr int kKChunk = 256;   // C values reduced by one partial sum
constexpr int kMaxTok = 2048;  // tokens per pass of the two kernels

template <typename T>
__device__ __forceinline__ void load16(const T* src, int n_avail, T* dst) {
  // 16 bytes of T from global into LDS; the ragged / unaligned case element by element
  constexpr int kVec = 16 / sizeof(T);
  if (n_avail >= kVec && (reinterpret_cast<uintptr_t>(src) & 15u) == 0) {
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  } else {
    for (int u = 0; u < kVec; ++u) dst[u] = u < n_avail ? src[u] : T{};
  }
}

template <typename T>
__global__ __launch_bounds__(256) void append_project(const T* __restrict__ x,
                                                      const T* __restrict__ w_dkv,
                                                      const T* __restrict__ w_kr, int n_tok,
                                                      int C, int d_c, int d_r, int k_chunk,
                                                      float* __restrict__ y_part) {
  // One workgroup: 64 output columns x one k_chunk-wide range of C x up to 16 tokens. Weights
  // and activations are staged through LDS with 16-byte loads issued together; thread (column
  // c, quarter kq) sums a quarter of the range for every token, and the quarters are added in
  // a fixed order through LDS.
  constexpr int kVec = 16 / sizeof(T);
  __shared__ __attribute__((aligned(16))) T xs[kTokTile][kKStage];
  __shared__ __attribute__((aligned(16))) T wsm[kKStage][kColTile];
  __shared__ float part[4][kTokTile][kColTile];
  const int ncols = d_c + d_r;
  const int c0 = blockIdx.x * kColTile;
  const int ks = blockIdx.y;
  const int n0 = blockIdx.z * kTokTile;
  const int ntok = min(kTokTile, n_tok - n0);
  const int k0 = ks * k_chunk, k1 = min(C, k0 + k_chunk);
  const int kn = k1 - k0;
  for (int e = threadIdx.x; e < ntok * (kKStage / kVec); e += 256) {
    const int r = e / (kKStage / kVec), kv = (e % (kKStage / kVec)) * kVec;
    load16(x + static_cast<int64_t>(n0 + r) * C + k0 + kv, kn - kv, &xs[r][kv]);
  }
  for (int e = threadIdx.x; e < kKStage * (kColTile / kVec); e += 256) {
    const int k = e / (kColTile / kVec), cv = (e % (kColTile / kVec)) * kVec;
    const int kg = k0 + k, cg = c0 + cv;
    if (k >= kn || cg >= ncols) {
      for (int u = 0; u < kVec; ++u) wsm[k][cv + u] = T{};
    } else if (cg < d_c) {
      load16(w_dkv + static_cast<int64_t>(kg) * d_c + cg, d_c - cg, &wsm[k][cv]);
    } else {
      load16(w_kr + static_cast<int64_t>(kg) * d_r + (cg - d_c), ncols - cg, &wsm[k][cv]);
    }
  }
  __syncthreads();
  const int c = threadIdx.x & 63, kq = threadIdx.x >> 6;
  const int kb = kq * (kKStage / 4), ke = min(kn, kb + kKStage / 4);
  float acc[kTokTile];
#pragma unroll
  for (int r = 0; r < kTokTile; ++r) acc[r] = 0.f;
  for (int k = kb; k < ke; ++k) {
    const float wv = ld(&wsm[k][0], c);
#pragma unroll
    for (int r = 0; r < kTokTile; ++r)
      if (r < ntok) acc[r] += ld(&xs[r][0], k) * wv;
  }
#pragma unroll
  for (int r = 0; r < kTokTile; ++r)
    if (r < ntok) part[kq][r][c] = acc[r];
  __syncthreads();
  for (int e = threadIdx.x; e < ntok * kColTile; e += 256) {
    const int r = e / kColTile, cc = e % kColTile;
    const int col = c0 + cc;
    if (col >= ncols) continue;
    const float y = ((part[0][r][cc] + part[1][r][cc]) + part[2][r][cc]) + part[3][r][cc];
    y_part[(static_cast<int64_t>(ks) * n_tok + n0 + r) * ncols + col] = y;
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
    // partial sums added in the fixed order k = 0, 1, ...; loads issued eight at a time
    float y = 0.f;
    int k = 0;
    for (; k + 8 <= n_ksplit; k += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = y_part[(static_cast<int64_t>(k + u) * n_tok + n) * ncols + c];
#pragma unroll
      for (int u = 0; u < 8; ++u) y += v[u];
    }
    for (; k < n_ksplit; ++k) y += y_part[(static_cast<int64_t>(k) * n_tok + n) * ncols + c];
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
  // Fixed 256-wide ranges of C per partial sum, added in a fixed order: a row's result does
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
