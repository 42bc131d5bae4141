// mla_cache_append: c = RMSNorm(x · W_DKV) * gamma, k_r = RoPE(x · W_KR, pos), written as one
// [c || k_r] row into the paged latent cache (Smallem article 13, "L'idée : garder un résumé",
// "L'obstacle : RoPE" and the cache extension in "Le code").
//
// Two kernels: a split-K projection of x against [W_DKV | W_KR] into fp32 partial sums (the
// projection is bound by reading the 2*C*(d_c+d_r)-byte weights, so it is spread over many
// workgroups even for a handful of tokens), then one workgroup per token that sums the
// partials in a fixed order, normalises, rotates and stores the row at its slot.
#include "absorb_tile.hpp"
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
__device__ __forceinline__ uint4 load16(const T* src, int n_avail) {
  // 16 bytes of T; the ragged or unaligned case element by element (missing ones are zero)
  constexpr int kVec = 16 / sizeof(T);
  if (n_avail >= kVec && (reinterpret_cast<uintptr_t>(src) & 15u) == 0)
    return *reinterpret_cast<const uint4*>(src);
  union {
    uint4 v;
    T e[kVec];
  } u;
  u.v = make_uint4(0u, 0u, 0u, 0u);
  for (int i = 0; i < kVec; ++i)
    if (i < n_avail) u.e[i] = src[i];
  return u.v;
}

template <typename T>
__global__ __launch_bounds__(256) void append_project(const T* __restrict__ x,
                                                      const T* __restrict__ w_a,
                                                      const T* __restrict__ w_b, int n_tok,
                                                      int C, int n_a, int n_b, int k_chunk,
                                                      float* __restrict__ y_part) {
  // One workgroup: 64 output columns x one k_chunk-wide range of C x up to 16 tokens. Weights
  // and activations are staged through LDS with 16-byte loads issued together; thread (column
  // c, quarter kq) sums a quarter of the range for every token, and the quarters are added in
  // a fixed order through LDS.
  constexpr int kVec = 16 / sizeof(T);
  __shared__ __attribute__((aligned(16))) T xs[kTokTile][kKStage];
  __shared__ __attribute__((aligned(16))) T wsm[kKStage][kColTile];
  __shared__ float part[4][kTokTile][kColTile];
  const int ncols = n_a + n_b;
  const int c0 = blockIdx.x * kColTile;
  const int ks = blockIdx.y;
  const int n0 = blockIdx.z * kTokTile;
  const int ntok = min(kTokTile, n_tok - n0);
  const int k0 = ks * k_chunk, k1 = min(C, k0 + k_chunk);
  const int kn = k1 - k0;
  // every 16-byte load of the stage is issued before the first LDS store
  constexpr int kXIt = kTokTile * (kKStage / kVec) / 256;   // 2 (bf16) or 4 (fp32)
  constexpr int kWIt = kKStage * (kColTile / kVec) / 256;   // 8 (bf16) or 16 (fp32)
  uint4 xr[kXIt], wr[kWIt];
#pragma unroll
  for (int i = 0; i < kXIt; ++i) {
    const int e = threadIdx.x + 256 * i;
    const int r = e / (kKStage / kVec), kv = (e % (kKStage / kVec)) * kVec;
    xr[i] = r < ntok ? load16(x + static_cast<int64_t>(n0 + r) * C + k0 + kv, kn - kv)
                     : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int i = 0; i < kWIt; ++i) {
    const int e = threadIdx.x + 256 * i;
    const int k = e / (kColTile / kVec), cv = (e % (kColTile / kVec)) * kVec;
    const int kg = k0 + k, cg = c0 + cv;
    if (k >= kn || cg >= ncols)
      wr[i] = make_uint4(0u, 0u, 0u, 0u);
    else if (cg < n_a)
      wr[i] = load16(w_a + static_cast<int64_t>(kg) * n_a + cg, n_a - cg);
    else
      wr[i] = load16(w_b + static_cast<int64_t>(kg) * n_b + (cg - n_a), ncols - cg);
  }
#pragma unroll
  for (int i = 0; i < kXIt; ++i) {
    const int e = threadIdx.x + 256 * i;
    const int r = e / (kKStage / kVec), kv = (e % (kKStage / kVec)) * kVec;
    *reinterpret_cast<uint4*>(&xs[r][kv]) = xr[i];
  }
#pragma unroll
  for (int i = 0; i < kWIt; ++i) {
    const int e = threadIdx.x + 256 * i;
    const int k = e / (kColTile / kVec), cv = (e % (kColTile / kVec)) * kVec;
    *reinterpret_cast<uint4*>(&wsm[k][cv]) = wr[i];
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

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kWtStride = kKStage * 2 + 16;  // bytes per transposed weight column in LDS

// The two projection kernels compute the split-K partial sums of y = x · [W_a | W_b] (columns
// 0 .. n_a - 1 from W_a [K, n_a], then n_b from W_b [K, n_b]; W_b may be absent with n_b = 0):
// the append's [W_DKV | W_KR], and the decode layer's query and output projections.
//
// bf16 projection on matrix cores, same partial sums as append_project (fixed 256-wide
// ranges of C, so a row's bits do not depend on the other tokens appended with it). One
// workgroup per (64 output columns, 256-wide range of C, 32 tokens); wave w computes the
// 32 columns 32 (w & 1) .. for the half (w >> 1) of the range, and the two halves are added
// in that order through LDS.
//  * A operand (tokens x k): rows of x, 16 bytes per lane straight from memory;
//  * B operand (k x columns): the weight tile is staged in LDS transposed (column-major, rows
//    padded to 528 bytes), so each lane's 8 consecutive k of one column are one 16-byte read.
__device__ inline void project_tile_mfma(const uint16_t* __restrict__ x,
                                         const uint16_t* __restrict__ w_a,
                                         const uint16_t* __restrict__ w_b, int n_tok, int C,
                                         int n_a, int n_b, float* __restrict__ y_part, int cbk,
                                         int ks, int n0) {
  __shared__ __attribute__((aligned(16))) char wt[kColTile * kWtStride];
  __shared__ float half1[2][16][64];
  const int ncols = n_a + n_b;
  const int c0 = cbk * kColTile;
  const int k0 = ks * kKStage;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int cb = w & 1, kh = w >> 1;
  // x fragments first (they do not depend on the staging)
  const int n = n0 + l32;
  bf16x8 af[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    const int k = k0 + 128 * kh + 16 * st + 8 * hi;
    af[st] = bf16x8{};
    if (n < n_tok && k + 8 <= C)
      af[st] = *reinterpret_cast<const bf16x8*>(x + static_cast<int64_t>(n) * C + k);
  }
  // weight tile [256 k x 64 columns]: 16-byte loads (8 columns of one k), all in flight,
  // then scattered into the transposed LDS layout
  uint4 wr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = threadIdx.x + 256 * i;
    const int k = e >> 3, cv = (e & 7) * 8;
    const int kg = k0 + k, cg = c0 + cv;
    wr[i] = make_uint4(0u, 0u, 0u, 0u);
    if (kg < C && cg < ncols) {
      const uint16_t* src = cg < n_a ? w_a + static_cast<int64_t>(kg) * n_a + cg
                                     : w_b + static_cast<int64_t>(kg) * n_b + (cg - n_a);
      wr[i] = *reinterpret_cast<const uint4*>(src);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = threadIdx.x + 256 * i;
    const int k = e >> 3, cv = (e & 7) * 8;
    const uint32_t v[4] = {wr[i].x, wr[i].y, wr[i].z, wr[i].w};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint16_t b = static_cast<uint16_t>(u & 1 ? v[u >> 1] >> 16 : v[u >> 1] & 0xffffu);
      *reinterpret_cast<uint16_t*>(wt + (cv + u) * kWtStride + 2 * k) = b;
    }
  }
  __syncthreads();
  f32x16 acc = {};
  const char* bcol = wt + (32 * cb + l32) * kWtStride + 2 * (128 * kh + 8 * hi);
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    const bf16x8 bf = *reinterpret_cast<const bf16x8*>(bcol + 32 * st);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[st], bf, acc, 0, 0, 0);
  }
  // D register r holds token 8 (r / 4) + 4 hi + r % 4, column l32
  if (kh == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) half1[cb][r][lane] = acc[r];
  }
  __syncthreads();
  if (kh == 0) {
    const int col = c0 + 32 * cb + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tok = n0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (tok < n_tok && col < ncols)
        y_part[(static_cast<int64_t>(ks) * n_tok + tok) * ncols + col] = acc[r] + half1[cb][r][lane];
    }
  }
}

__global__ __launch_bounds__(256) void append_project_mfma(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ w_a,
                                                           const uint16_t* __restrict__ w_b,
                                                           int n_tok, int C, int n_a, int n_b,
                                                           float* __restrict__ y_part) {
  project_tile_mfma(x, w_a, w_b, n_tok, C, n_a, n_b, y_part, blockIdx.x, blockIdx.y,
                    blockIdx.z * 32);
}

// kFp8: the row goes out as e4m3 bytes (cache8) and its scale (scale8), quantised from the
// values the bf16 row would hold.
template <typename T, bool kFp8>
__global__ __launch_bounds__(1024) void append_finalize(
    const float* __restrict__ y_part, int n_ksplit, int n_tok, const T* __restrict__ gamma,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ table, int batch, int max_blocks, int num_blocks, int bs,
    int d_c, int d_r, float eps, float base, T* __restrict__ cache, uint8_t* __restrict__ cache8,
    float* __restrict__ scale8) {
  extern __shared__ float ys[];  // [d_c + d_r]
  __shared__ float red[64];
  const int n = blockIdx.x;
  const int ncols = d_c + d_r;
  const int lat_blocks = cdiv(d_c, kColTile);  // 64-column blocks of the latent part
  // the row's slot first: its dependent loads (sequence, position, block table) overlap the
  // partial sums below
  const int b = seq_idx[n], p = pos[n];
  const int64_t slot = (b < 0 || b >= batch) ? -1 : cache_slot(table, max_blocks, bs, num_blocks, b, p);
  // blockDim.x is a multiple of 64: pass c0 gives wave w the 64-column block c0 / 64 + w
  for (int c0 = 0; c0 < ncols; c0 += blockDim.x) {
    const int c = c0 + static_cast<int>(threadIdx.x);
    float y = 0.f;
    if (c < ncols) {
      // partial sums added in the fixed order k = 0, 1, ...; up to 32 loads in flight
      for (int k = 0; k < n_ksplit; k += 32) {
        float v[32];
#pragma unroll
        for (int u = 0; u < 32; ++u)
          v[u] = k + u < n_ksplit ? y_part[(static_cast<int64_t>(k + u) * n_tok + n) * ncols + c] : 0.f;
#pragma unroll
        for (int u = 0; u < 32; ++u)
          if (k + u < n_ksplit) y += v[u];
      }
      ys[c] = y;
    }
    // sum of squares of the latent part: each 64-column block by a butterfly over its wave
    // (a fixed order, independent of the block size), then the blocks in order below
    const int blk = c0 / 64 + static_cast<int>(threadIdx.x >> 6);
    if (blk < lat_blocks) {
      const float s2 = wave_sum(c < d_c ? square_rn(y) : 0.f);
      if ((threadIdx.x & 63) == 0) red[blk] = s2;
    }
  }
  __syncthreads();
  float ss = 0.f;
  for (int j = 0; j < lat_blocks; ++j) ss += red[j];
  if (slot < 0) return;
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(d_c) + eps);
  if constexpr (kFp8) {
    // the row rounded to bf16 in place (each thread rewrites only the columns it reads)
    float amax = 0.f;
    for (int c = threadIdx.x; c < d_c; c += blockDim.x) {
      const float v = bf16_to_f32(f32_to_bf16(ys[c] * inv * ld(gamma, c)));
      ys[c] = v;
      amax = fmaxf(amax, fabsf(v));
    }
    for (int j = threadIdx.x; j < d_r / 2; j += blockDim.x) {
      float cs, sn;
      rope_cos_sin(p, j, d_r, base, &cs, &sn);
      const float a = ys[d_c + 2 * j], q = ys[d_c + 2 * j + 1];
      float u, v;
      rope_rotate(a, q, cs, sn, &u, &v);
      u = bf16_to_f32(f32_to_bf16(u));
      v = bf16_to_f32(f32_to_bf16(v));
      ys[d_c + 2 * j] = u;
      ys[d_c + 2 * j + 1] = v;
      amax = fmaxf(amax, fmaxf(fabsf(u), fabsf(v)));
    }
    amax = block_max(amax, red);  // its barriers also publish the rounded row
    const int e = e4m3_scale_exp(amax);
    const float rs = ldexpf(1.f, -e);
    unsigned* out = reinterpret_cast<unsigned*>(cache8 + slot * ncols);
    for (int i = threadIdx.x; i < ncols / 4; i += blockDim.x)
      out[i] = e4m3_pack4(ys[4 * i] * rs, ys[4 * i + 1] * rs, ys[4 * i + 2] * rs,
                          ys[4 * i + 3] * rs);
    if (threadIdx.x == 0) scale8[slot] = ldexpf(1.f, e);
    return;
  }
  T* row = cache + slot * ncols;
  for (int c = threadIdx.x; c < d_c; c += blockDim.x) st(row, c, ys[c] * inv * ld(gamma, c));
  for (int j = threadIdx.x; j < d_r / 2; j += blockDim.x) {
    float cs, sn;
    rope_cos_sin(p, j, d_r, base, &cs, &sn);
    const float a = ys[d_c + 2 * j], q = ys[d_c + 2 * j + 1];
    float u, v;
    rope_rotate(a, q, cs, sn, &u, &v);
    st(row, d_c + 2 * j, u);
    st(row, d_c + 2 * j + 1, v);
  }
}

// Rows of bf16 values to e4m3 bytes and scales, one wave per row (the rule of append_finalize).
__global__ __launch_bounds__(256) void quantize_rows_e4m3(const uint16_t* __restrict__ rows,
                                                         int64_t n_rows, int ncols,
                                                         uint8_t* __restrict__ out,
                                                         float* __restrict__ scale) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= n_rows) return;
  const int ng = ncols / 4;  // groups of four values
  const uint2* src = reinterpret_cast<const uint2*>(rows + r * ncols);
  constexpr int kMaxG = 4;   // ncols <= 1024
  uint2 v[kMaxG];
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxG; ++k) {
    const int g = lane + 64 * k;
    v[k] = g < ng ? src[g] : make_uint2(0u, 0u);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bf16_to_f32(v[k].x & 0xffffu)),
                                   fabsf(bf16_to_f32(v[k].x >> 16))),
                             fmaxf(fabsf(bf16_to_f32(v[k].y & 0xffffu)),
                                   fabsf(bf16_to_f32(v[k].y >> 16)))));
  }
  amax = wave_max(amax);
  const int e = e4m3_scale_exp(amax);
  const float rs = ldexpf(1.f, -e);
  unsigned* dst = reinterpret_cast<unsigned*>(out + r * ncols);
#pragma unroll
  for (int k = 0; k < kMaxG; ++k) {
    const int g = lane + 64 * k;
    if (g < ng)
      dst[g] = e4m3_pack4(bf16_to_f32(v[k].x & 0xffffu) * rs, bf16_to_f32(v[k].x >> 16) * rs,
                          bf16_to_f32(v[k].y & 0xffffu) * rs, bf16_to_f32(v[k].y >> 16) * rs);
  }
  if (lane == 0) scale[r] = ldexpf(1.f, e);
}

// ---- the append's projection and the query absorption of a decode step in one launch.
//
// Both are weight streams with no dependency on each other (W_DKV | W_KR for the new tokens,
// W_UK for the queries), each too small to fill the chip for long: run as one grid, the
// absorb tiles fill the CUs the projection leaves idle and the step saves a launch. The
// append's finalize (sum of the partials in k order, RMSNorm, RoPE, store) follows as before.
template <int kKS>
__global__ __launch_bounds__(256) void project_absorb(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ w_a,
                                                      const uint16_t* __restrict__ w_b,
                                                      int n_tok, int C, int n_a, int n_b,
                                                      float* __restrict__ y_part, int col_blocks,
                                                      int n_ksplit, AbsorbArgs q, int absorb_rb,
                                                      int absorb_zb) {
  const int n_proj = col_blocks * n_ksplit * cdiv(n_tok, 32);
  if (static_cast<int>(blockIdx.x) >= n_proj) {
    // an absorb tile: z fastest, then the 32-row block, then the head
    int t = blockIdx.x - n_proj;
    const int z = t % absorb_zb;
    t /= absorb_zb;
    absorb_tile_mfma<kKS>(q, t / absorb_rb, (t % absorb_rb) * 32, z, absorb_zb);
    return;
  }
  const int t = blockIdx.x;
  const int cb = t % col_blocks, ks = (t / col_blocks) % n_ksplit, nt = t / (col_blocks * n_ksplit);
  project_tile_mfma(x, w_a, w_b, n_tok, C, n_a, n_b, y_part, cb, ks, 32 * nt);
}

// Token n of a decode step: sequence n / s_q, position seq_lens[n / s_q] - s_q + n % s_q.
__global__ __launch_bounds__(256) void step_positions(int n_tok, int s_q,
                                                      const int32_t* __restrict__ seq_lens,
                                                      int32_t* __restrict__ seq_idx,
                                                      int32_t* __restrict__ pos) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= n_tok) return;
  const int b = n / s_q;
  seq_idx[n] = b;
  pos[n] = seq_lens[b] - s_q + (n - b * s_q);
}

// project_absorb built for the absorbed queries' K-steps: 8 (D <= 128) or 16.
void launch_project_absorb(const mla_dims& d, dim3 grid, hipStream_t s, const void* x,
                           const void* w_dkv, const void* w_kr, int n, float* y_part,
                           const AppendPlan& p, const AbsorbArgs& q, int rb, int zb) {
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* wa = static_cast<const uint16_t*>(w_dkv);
  const auto* wb = static_cast<const uint16_t*>(w_kr);
  if (d.d_nope <= 128)
    hipLaunchKernelGGL(project_absorb<8>, grid, dim3(256), 0, s, xp, wa, wb, n, d.d_model, d.d_c,
                       d.d_r, y_part, p.col_blocks, p.n_ksplit, q, rb, zb);
  else
    hipLaunchKernelGGL(project_absorb<16>, grid, dim3(256), 0, s, xp, wa, wb, n, d.d_model,
                       d.d_c, d.d_r, y_part, p.col_blocks, p.n_ksplit, q, rb, zb);
}

}  // namespace

int projection_ksplit(int K) { return cdiv(K, kKChunk); }

bool step_project_fits(const mla_dims& d, int n_tok) {
  return d.dtype == MLA_BF16 && !(d.flags & MLA_FLAG_GENERIC_KERNELS) && d.d_model % 8 == 0 &&
         d.d_c % 8 == 0 && d.d_r % 8 == 0 && absorb_mfma_fits(d) && n_tok >= 1 &&
         n_tok <= kMaxTok;
}

hipError_t launch_step_project(const mla_dims& d, int batch, int s_q, const void* x,
                               const void* w_dkv, const void* w_kr, float* y_part,
                               const void* q_nope, const void* q_pe, const int32_t* seq_lens,
                               const void* w_uk, void* q_abs, hipStream_t s) {
  const int n = batch * s_q;
  const AppendPlan p = append_plan(d, n);
  AbsorbArgs q = absorb_args(d, n, q_nope, q_pe, nullptr, w_uk, q_abs);
  q.lens = seq_lens;
  q.s_q = s_q;
  int rb = 1, zb = 1;
  const int tiles = absorb_tiles(q, &rb, &zb);
  const int proj = p.col_blocks * p.n_ksplit * cdiv(n, 32);
  launch_project_absorb(d, dim3(proj + tiles), s, x, w_dkv, w_kr, n, y_part, p, q, rb, zb);
  return hipGetLastError();
}

hipError_t launch_step_positions(int batch, int s_q, const int32_t* seq_lens, int32_t* seq_idx,
                                 int32_t* pos, hipStream_t s) {
  const int n = batch * s_q;
  hipLaunchKernelGGL(step_positions, dim3(cdiv(n, 256)), dim3(256), 0, s, n, s_q, seq_lens,
                     seq_idx, pos);
  return hipGetLastError();
}

hipError_t launch_projection_partials(int dt, bool mfma, int n_tok, int K, const void* x,
                                      const void* w_a, int n_a, const void* w_b, int n_b,
                                      float* y_part, hipStream_t s) {
  const int ncols = n_a + n_b;
  const int n_ksplit = projection_ksplit(K);
  if (dt == MLA_BF16 && mfma) {
    hipLaunchKernelGGL(append_project_mfma, dim3(cdiv(ncols, kColTile), n_ksplit, cdiv(n_tok, 32)),
                       dim3(256), 0, s, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(w_a), static_cast<const uint16_t*>(w_b), n_tok,
                       K, n_a, n_b, y_part);
  } else if (dt == MLA_BF16) {
    hipLaunchKernelGGL(append_project<bf16>, dim3(cdiv(ncols, kColTile), n_ksplit, cdiv(n_tok, kTokTile)),
                       dim3(256), 0, s, static_cast<const bf16*>(x), static_cast<const bf16*>(w_a),
                       static_cast<const bf16*>(w_b), n_tok, K, n_a, n_b, kKChunk, y_part);
  } else {
    hipLaunchKernelGGL(append_project<float>, dim3(cdiv(ncols, kColTile), n_ksplit, cdiv(n_tok, kTokTile)),
                       dim3(256), 0, s, static_cast<const float*>(x), static_cast<const float*>(w_a),
                       static_cast<const float*>(w_b), n_tok, K, n_a, n_b, kKChunk, y_part);
  }
  return hipGetLastError();
}

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

hipError_t launch_quantize_e4m3(int64_t n_rows, int ncols, const void* rows, void* out,
                               float* scale, hipStream_t s) {
  const int64_t nb = (n_rows + 3) / 4;
  for (int64_t b0 = 0; b0 < nb; b0 += 0x7fffffff) {
    const int64_t n = nb - b0 < 0x7fffffff ? nb - b0 : 0x7fffffff;
    const int64_t r0 = b0 * 4;
    hipLaunchKernelGGL(quantize_rows_e4m3, dim3(static_cast<unsigned>(n)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(rows) + r0 * ncols, n_rows - r0, ncols,
                       static_cast<uint8_t*>(out) + r0 * ncols, scale + r0);
  }
  return hipGetLastError();
}

size_t append_ws_bytes(const mla_dims& d, int n_tok) {
  const AppendPlan p = append_plan(d, n_tok);
  const size_t n = n_tok < kMaxTok ? n_tok : kMaxTok;
  return static_cast<size_t>(p.n_ksplit) * n * (d.d_c + d.d_r) * sizeof(float);
}

hipError_t launch_append(const mla_dims& d, int n_tok, const void* x, const int32_t* seq_idx,
                         const int32_t* pos, const void* w_dkv, const void* gamma,
                         const void* w_kr, const int32_t* table, int batch, int max_blocks,
                         int num_blocks, void* cache, float* cache_scale, void* ws,
                         hipStream_t s) {
  return launch_append_absorb(d, n_tok, x, seq_idx, pos, w_dkv, gamma, w_kr, table, batch,
                              max_blocks, num_blocks, cache, cache_scale, ws, 0, 0, nullptr,
                              nullptr, nullptr, nullptr, nullptr, s);
}

hipError_t launch_append_absorb(const mla_dims& d, int n_tok, const void* x,
                                const int32_t* seq_idx, const int32_t* pos, const void* w_dkv,
                                const void* gamma, const void* w_kr, const int32_t* table,
                                int batch, int max_blocks, int num_blocks, void* cache,
                                float* cache_scale, void* ws, int q_batch, int s_q, const void* q_nope, const void* q_pe,
                                const int32_t* q_pos, const void* w_uk, void* q_abs,
                                hipStream_t s) {
  float* y_part = static_cast<float*>(ws);
  const size_t lds = static_cast<size_t>(d.d_c + d.d_r) * sizeof(float);
  const size_t elt = d.dtype == MLA_BF16 ? 2 : 4;
  const int ncols = d.d_c + d.d_r;
  const dim3 fin_block(ncols >= 1024 ? 1024 : (ncols + 63) / 64 * 64);
  // matrix-core projection: every 16-byte weight and activation load stays inside one row
  // and one of the two weight matrices (16-byte-aligned base pointers are a library rule)
  const bool mfma_ok = d.dtype == MLA_BF16 && !(d.flags & MLA_FLAG_GENERIC_KERNELS) &&
                       d.d_model % 8 == 0 && d.d_c % 8 == 0 && d.d_r % 8 == 0;
  const int M = q_batch * s_q;
  // the absorption rides along with the first pass of the projection where both run on the
  // matrix cores; otherwise it is launched on its own after the append
  bool absorb_pending = M > 0;
  for (int t0 = 0; t0 < n_tok; t0 += kMaxTok) {
    const int n = n_tok - t0 < kMaxTok ? n_tok - t0 : kMaxTok;
    const AppendPlan p = append_plan(d, n);
    const dim3 g1(p.col_blocks, p.n_ksplit, p.tok_tiles);
    const void* xc = static_cast<const char*>(x) + static_cast<size_t>(t0) * d.d_model * elt;
    if (d.dtype == MLA_BF16) {
      if (mfma_ok && absorb_pending && absorb_mfma_fits(d)) {
        const AbsorbArgs q = absorb_args(d, M, q_nope, q_pe, q_pos, w_uk, q_abs);
        int rb = 1, zb = 1;
        const int tiles = absorb_tiles(q, &rb, &zb);
        const int proj = p.col_blocks * p.n_ksplit * cdiv(n, 32);
        launch_project_absorb(d, dim3(proj + tiles), s, xc, w_dkv, w_kr, n, y_part, p, q, rb, zb);
        absorb_pending = false;
      } else if (mfma_ok) {
        hipLaunchKernelGGL(append_project_mfma, dim3(p.col_blocks, p.n_ksplit, cdiv(n, 32)),
                           dim3(256), 0, s, static_cast<const uint16_t*>(xc),
                           static_cast<const uint16_t*>(w_dkv), static_cast<const uint16_t*>(w_kr),
                           n, d.d_model, d.d_c, d.d_r, y_part);
      } else {
        hipLaunchKernelGGL(append_project<bf16>, g1, dim3(256), 0, s, static_cast<const bf16*>(xc),
                           static_cast<const bf16*>(w_dkv), static_cast<const bf16*>(w_kr), n,
                           d.d_model, d.d_c, d.d_r, p.k_chunk, y_part);
      }
      if (cache_scale != nullptr)
        hipLaunchKernelGGL((append_finalize<bf16, true>), dim3(n), fin_block, lds, s, y_part,
                           p.n_ksplit, n, static_cast<const bf16*>(gamma), seq_idx + t0, pos + t0,
                           table, batch, max_blocks, num_blocks, d.block_size, d.d_c, d.d_r,
                           d.rms_eps, d.rope_base, nullptr, static_cast<uint8_t*>(cache),
                           cache_scale);
      else
        hipLaunchKernelGGL((append_finalize<bf16, false>), dim3(n), fin_block, lds, s, y_part,
                           p.n_ksplit, n, static_cast<const bf16*>(gamma), seq_idx + t0, pos + t0,
                           table, batch, max_blocks, num_blocks, d.block_size, d.d_c, d.d_r,
                           d.rms_eps, d.rope_base, static_cast<bf16*>(cache), nullptr, nullptr);
    } else {
      hipLaunchKernelGGL(append_project<float>, g1, dim3(256), 0, s,
                         static_cast<const float*>(xc), static_cast<const float*>(w_dkv),
                         static_cast<const float*>(w_kr), n, d.d_model, d.d_c, d.d_r, p.k_chunk,
                         y_part);
      hipLaunchKernelGGL((append_finalize<float, false>), dim3(n), fin_block, lds, s, y_part,
                         p.n_ksplit, n, static_cast<const float*>(gamma), seq_idx + t0, pos + t0,
                         table, batch, max_blocks, num_blocks, d.block_size, d.d_c, d.d_r,
                         d.rms_eps, d.rope_base, static_cast<float*>(cache), nullptr, nullptr);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (absorb_pending) return launch_absorb(d, q_batch, s_q, q_nope, q_pe, q_pos, w_uk, q_abs, s);
  return hipSuccess;
}

}  // namespace mla
