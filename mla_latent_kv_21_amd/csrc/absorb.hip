// mla_absorb_q: q_abs = [q_nope_h · W_UK[:, g(h)]^T || RoPE(q_pe_h, pos)] (Smallem article 13,
// "Ce que DeepSeek fait de plus": the query is moved into latent space once per token, so the
// cached latents are never expanded; GQLA summary, section 2: W_UK is indexed by group).
//
// bf16 runs on matrix cores (absorb_mfma); the portable kernel (fp32, or other shapes) uses
// one workgroup per (head, 16 query rows): the head's d_c x D slice of W_UK is read once per
// 16 rows and every thread produces whole latent columns for all 16 rows.
#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kRows = 16;

template <typename T>
__global__ __launch_bounds__(256) void absorb_kernel(const T* __restrict__ q_nope,
                                                     const T* __restrict__ q_pe,
                                                     const int32_t* __restrict__ q_pos,
                                                     const T* __restrict__ w_uk, int M, int H,
                                                     int G, int D, int d_c, int d_r, float base,
                                                     T* __restrict__ q_abs) {
  extern __shared__ float qs[];  // [kRows][D]
  const int h = blockIdx.x;
  const int g = h / (H / G);
  const int m0 = blockIdx.y * kRows;
  const int row = d_c + d_r;
  for (int e = threadIdx.x; e < kRows * D; e += blockDim.x) {
    const int r = e / D, k = e % D;
    const int m = m0 + r;
    qs[e] = m < M ? ld(q_nope, (static_cast<int64_t>(m) * H + h) * D + k) : 0.f;
  }
  __syncthreads();
  const int64_t ldw = static_cast<int64_t>(G) * D;
  for (int j = threadIdx.x; j < d_c; j += blockDim.x) {
    float acc[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) acc[r] = 0.f;
    const T* wrow = w_uk + j * ldw + static_cast<int64_t>(g) * D;
    for (int k = 0; k < D; ++k) {
      const float w = ld(wrow, k);
#pragma unroll
      for (int r = 0; r < kRows; ++r) acc[r] += qs[r * D + k] * w;
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int m = m0 + r;
      if (m < M) st(q_abs, (static_cast<int64_t>(m) * H + h) * row + j, acc[r]);
    }
  }
  const int half = d_r / 2;
  for (int e = threadIdx.x; e < kRows * half; e += blockDim.x) {
    const int r = e / half, j = e % half;
    const int m = m0 + r;
    if (m >= M) continue;
    float cs, sn;
    rope_cos_sin(q_pos[m], j, d_r, base, &cs, &sn);
    const int64_t src = (static_cast<int64_t>(m) * H + h) * d_r + 2 * j;
    const float a = ld(q_pe, src), b = ld(q_pe, src + 1);
    const int64_t dst = (static_cast<int64_t>(m) * H + h) * row + d_c + 2 * j;
    st(q_abs, dst, a * cs - b * sn);
    st(q_abs, dst + 1, a * sn + b * cs);
  }
}

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

// bf16 absorption on matrix cores: per head, Q_lat[32 rows x d_c] = q_nope[32 x D] ·
// W_UK[:, g]^T, i.e. a product whose operands are both contiguous along the contraction
// (rows of q_nope and rows of W_UK), so MFMA fragments load straight from memory. One
// workgroup per (head, 32 rows, 128 latent columns); wave w computes one 32-column block.
__global__ __launch_bounds__(256) void absorb_mfma(const uint16_t* __restrict__ q_nope,
                                                   const uint16_t* __restrict__ q_pe,
                                                   const int32_t* __restrict__ q_pos,
                                                   const uint16_t* __restrict__ w_uk, int M,
                                                   int H, int G, int D, int d_c, int d_r,
                                                   float base, uint16_t* __restrict__ q_abs) {
  const int h = blockIdx.x, m0 = blockIdx.y * 32;
  const int g = h / (H / G);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int row = d_c + d_r;
  const int ksteps = D / 16;  // at most 16 (D <= 256)
  const int m = m0 + l32;
  bf16x8 af[16];
  const bf16x8 zero = {};
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    af[ks] = zero;
    if (ks < ksteps && m < M)
      af[ks] = *reinterpret_cast<const bf16x8*>(q_nope + (static_cast<int64_t>(m) * H + h) * D +
                                                16 * ks + 8 * hi);
  }
  const int64_t ldw = static_cast<int64_t>(G) * D;
  // B fragments of one 32-column block: all requested before the first MFMA
  bf16x8 bv[16];
  auto load_b = [&](int nb) __attribute__((always_inline)) {
    const uint16_t* wr = w_uk + (nb * 32 + l32) * ldw + static_cast<int64_t>(g) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      bv[ks] = ks < ksteps ? *reinterpret_cast<const bf16x8*>(wr + 16 * ks) : zero;
  };
  int nb = 4 * blockIdx.z + w;
  const int nb_end = min(d_c / 32, 4 * static_cast<int>(blockIdx.z) + 4);
  if (nb < nb_end) load_b(nb);

  // rotary part, while the first block's fragments are in flight: the (row, pair) items are
  // shared out over the z-blocks of this head
  const int half = d_r / 2;
  for (int e = threadIdx.x + blockIdx.z * blockDim.x; e < 32 * half; e += blockDim.x * gridDim.z) {
    const int r = e / half, jj = e % half;
    const int mm = m0 + r;
    if (mm >= M) continue;
    float cs, sn;
    rope_cos_sin(q_pos[mm], jj, d_r, base, &cs, &sn);
    const int64_t src = (static_cast<int64_t>(mm) * H + h) * d_r + 2 * jj;
    const float x0 = bf16_to_f32(q_pe[src]), x1 = bf16_to_f32(q_pe[src + 1]);
    const int64_t dst = (static_cast<int64_t>(mm) * H + h) * row + d_c + 2 * jj;
    q_abs[dst] = f32_to_bf16(x0 * cs - x1 * sn);
    q_abs[dst + 1] = f32_to_bf16(x0 * sn + x1 * cs);
  }

  while (nb < nb_end) {
    const int j = nb * 32 + l32;
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      if (ks < ksteps) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], bv[ks], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int mm = m0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (mm < M) q_abs[(static_cast<int64_t>(mm) * H + h) * row + j] = f32_to_bf16(acc[r]);
    }
    nb += 4;
    if (nb < nb_end) load_b(nb);
  }
}

}  // namespace

hipError_t launch_absorb(const mla_dims& d, int batch, int s_q, const void* q_nope,
                         const void* q_pe, const int32_t* q_pos, const void* w_uk, void* q_abs,
                         hipStream_t s) {
  const int M = batch * s_q;
  if (d.dtype == MLA_BF16 && !(d.flags & MLA_FLAG_GENERIC_KERNELS) && d.d_c % 32 == 0 &&
      d.d_nope % 16 == 0 && d.d_nope <= 256) {
    hipLaunchKernelGGL(absorb_mfma, dim3(d.n_heads, cdiv(M, 32), cdiv(d.d_c / 32, 4)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_pe),
                       q_pos, static_cast<const uint16_t*>(w_uk), M, d.n_heads, d.n_groups,
                       d.d_nope, d.d_c, d.d_r, d.rope_base, static_cast<uint16_t*>(q_abs));
    return hipGetLastError();
  }
  const dim3 grid(d.n_heads, cdiv(M, kRows));
  const size_t lds = static_cast<size_t>(kRows) * d.d_nope * sizeof(float);
  if (d.dtype == MLA_BF16) {
    hipLaunchKernelGGL(absorb_kernel<bf16>, grid, dim3(256), lds, s,
                       static_cast<const bf16*>(q_nope), static_cast<const bf16*>(q_pe), q_pos,
                       static_cast<const bf16*>(w_uk), M, d.n_heads, d.n_groups, d.d_nope, d.d_c,
                       d.d_r, d.rope_base, static_cast<bf16*>(q_abs));
  } else {
    hipLaunchKernelGGL(absorb_kernel<float>, grid, dim3(256), lds, s,
                       static_cast<const float*>(q_nope), static_cast<const float*>(q_pe), q_pos,
                       static_cast<const float*>(w_uk), M, d.n_heads, d.n_groups, d.d_nope,
                       d.d_c, d.d_r, d.rope_base, static_cast<float*>(q_abs));
  }
  return hipGetLastError();
}

}  // namespace mla
