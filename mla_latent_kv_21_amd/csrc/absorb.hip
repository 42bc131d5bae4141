// mla_absorb_q: q_abs = [q_nope_h · W_UK[:, g(h)]^T || RoPE(q_pe_h, pos)] (Smallem article 13,
// "Ce que DeepSeek fait de plus": the query is moved into latent space once per token, so the
// cached latents are never expanded; GQLA summary, section 2: W_UK is indexed by group).
//
// bf16 runs on matrix cores (absorb_mfma); the portable kernel (fp32, or other shapes) uses
// one workgroup per (head, 16 query rows): the head's d_c x D slice of W_UK is read once per
// 16 rows and every thread produces whole latent columns for all 16 rows.
#include "absorb_tile.hpp"
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

// One workgroup per absorb tile (absorb_tile.hpp).
template <int kKS>
__global__ __launch_bounds__(256) void absorb_mfma(AbsorbArgs q) {
  absorb_tile_mfma<kKS>(q, blockIdx.x, blockIdx.y * 32, blockIdx.z, gridDim.z);
}

}  // namespace

bool absorb_mfma_fits(const mla_dims& d) {
  return d.dtype == MLA_BF16 && !(d.flags & MLA_FLAG_GENERIC_KERNELS) && d.d_c % 32 == 0 &&
         d.d_nope % 16 == 0 && d.d_nope <= 256;
}

AbsorbArgs absorb_args(const mla_dims& d, int M, const void* q_nope, const void* q_pe,
                       const int32_t* q_pos, const void* w_uk, void* q_abs) {
  AbsorbArgs q;
  q.q_nope = static_cast<const uint16_t*>(q_nope);
  q.q_pe = static_cast<const uint16_t*>(q_pe);
  q.q_pos = q_pos;
  q.lens = nullptr;
  q.s_q = 1;
  q.w_uk = static_cast<const uint16_t*>(w_uk);
  q.M = M; q.H = d.n_heads; q.G = d.n_groups; q.D = d.d_nope; q.d_c = d.d_c; q.d_r = d.d_r;
  q.base = d.rope_base;
  q.q_abs = static_cast<uint16_t*>(q_abs);
  return q;
}

hipError_t launch_absorb(const mla_dims& d, int batch, int s_q, const void* q_nope,
                         const void* q_pe, const int32_t* q_pos, const void* w_uk, void* q_abs,
                         hipStream_t s) {
  const int M = batch * s_q;
  if (absorb_mfma_fits(d)) {
    const AbsorbArgs q = absorb_args(d, M, q_nope, q_pe, q_pos, w_uk, q_abs);
    const dim3 grid(d.n_heads, cdiv(M, 32), cdiv(d.d_c / 32, 4));
    if (d.d_nope <= 128)
      hipLaunchKernelGGL(absorb_mfma<8>, grid, dim3(256), 0, s, q);
    else
      hipLaunchKernelGGL(absorb_mfma<16>, grid, dim3(256), 0, s, q);
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
