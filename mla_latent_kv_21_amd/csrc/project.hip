// The decode layer's projections on either side of the attention path (Smallem article 13,
// "Le code": query_down, query_norm, query_up and query_rope before it, proj after it):
//
//   mla_query_project:  c_q = RMSNorm(x · W_DQ) * gamma_q;  q_nope = c_q · W_UQ;  q_pe = c_q · W_QR
//   mla_output_project: y = o · W_O + b_O
//
// Each product is the append's split-K projection (fixed 256-wide ranges of K, partial sums
// added in a fixed order) followed by project_finalize, which sums the partials of one token
// and applies what the step needs: the RMSNorm and gain of query_down, the bias of proj, and
// the split of [W_UQ | W_QR]'s columns into q_nope and q_pe. Tokens go through in passes of at
// most kProjTok, which bounds the workspace.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kProjTok = 32;      // tokens per pass
constexpr int kFinCols = 256;     // columns per finalize workgroup when nothing couples them
constexpr int kFinThreads = 256;  // ... one column per thread
constexpr int kNormThreads = 1024;  // a normalised row: one workgroup per token

// Workgroup (token n, column chunk j) of one pass: y_c = sum_k y_part[k][n][c], k = 0, 1, ...
// (sixteen partial sums of a column requested at once: the sum is a chain of round trips).
// With n_norm > 0 the workgroup holds the whole row (one chunk) and applies
// y_c / sqrt(mean_{c' < n_norm} y_c'^2 + eps) * gamma_c to the first n_norm columns. bias
// (nullable) is added after. Columns c < n_a go to out_a (rows of n_a), the rest to out_b (rows
// of ncols - n_a).
template <typename T>
__global__ __launch_bounds__(kNormThreads) void project_finalize(
    const float* __restrict__ y_part, int n_ksplit, int n_tok, int ncols, int n_norm,
    const T* __restrict__ gamma, float eps, const T* __restrict__ bias, T* __restrict__ out_a,
    int n_a, T* __restrict__ out_b) {
  extern __shared__ float ys[];  // [ncols] when n_norm > 0
  __shared__ float red[16];
  const int n = blockIdx.x;
  const int c0 = n_norm > 0 ? 0 : blockIdx.y * kFinCols;
  const int c1 = n_norm > 0 ? ncols : min(ncols, c0 + kFinCols);
  const int n_b = ncols - n_a;
  auto sum_col = [&](int c) {
    // the partial sums of column c in the fixed order k = 0, 1, ...
    float y = 0.f;
    for (int k = 0; k < n_ksplit; k += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        v[u] = k + u < n_ksplit ? y_part[(static_cast<int64_t>(k + u) * n_tok + n) * ncols + c] : 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (k + u < n_ksplit) y += v[u];
    }
    return y;
  };
  auto put = [&](int c, float y) {
    if (bias != nullptr) y += ld(bias, c);
    if (c < n_a)
      st(out_a, static_cast<int64_t>(n) * n_a + c, y);
    else
      st(out_b, static_cast<int64_t>(n) * n_b + (c - n_a), y);
  };
  if (n_norm == 0) {
    for (int c = c0 + threadIdx.x; c < c1; c += blockDim.x) put(c, sum_col(c));
    return;
  }
  float ss = 0.f;
  for (int c = threadIdx.x; c < ncols; c += blockDim.x) {
    const float y = sum_col(c);
    ys[c] = y;
    if (c < n_norm) ss += y * y;
  }
  ss = block_sum(ss, red);  // also orders the ys writes before the reads below
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(n_norm) + eps);
  for (int c = threadIdx.x; c < ncols; c += blockDim.x)
    put(c, c < n_norm ? ys[c] * inv * ld(gamma, c) : ys[c]);
}

template <typename T>
hipError_t finalize(const float* y_part, int n_ksplit, int n, int ncols, int n_norm,
                    const void* gamma, float eps, const void* bias, void* out_a, int n_a,
                    void* out_b, hipStream_t s) {
  const dim3 grid(n, n_norm > 0 ? 1 : cdiv(ncols, kFinCols));
  const size_t lds = n_norm > 0 ? static_cast<size_t>(ncols) * sizeof(float) : 0;
  hipLaunchKernelGGL(project_finalize<T>, grid, dim3(n_norm > 0 ? kNormThreads : kFinThreads), lds,
                     s, y_part, n_ksplit, n,
                     ncols, n_norm, static_cast<const T*>(gamma), eps, static_cast<const T*>(bias),
                     static_cast<T*>(out_a), n_a, static_cast<T*>(out_b));
  return hipGetLastError();
}

hipError_t finalize_dt(int dt, const float* y_part, int n_ksplit, int n, int ncols,
                       int n_norm, const void* gamma, float eps, const void* bias, void* out_a,
                       int n_a, void* out_b, hipStream_t s) {
  return dt == MLA_BF16 ? finalize<bf16>(y_part, n_ksplit, n, ncols, n_norm, gamma, eps, bias,
                                         out_a, n_a, out_b, s)
                        : finalize<float>(y_part, n_ksplit, n, ncols, n_norm, gamma, eps, bias,
                                          out_a, n_a, out_b, s);
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// the matrix-core projection keeps every 16-byte load inside one row of one matrix
bool mfma_ok(const mla_dims& d, int K, int n_a, int n_b) {
  return d.dtype == MLA_BF16 && !(d.flags & MLA_FLAG_GENERIC_KERNELS) && K % 8 == 0 &&
         n_a % 8 == 0 && n_b % 8 == 0;
}

}  // namespace

size_t query_project_ws_bytes(const mla_dims& d, int n_tok, int d_q) {
  const size_t n = static_cast<size_t>(n_tok < kProjTok ? n_tok : kProjTok);
  const size_t elt = d.dtype == MLA_BF16 ? 2 : 4;
  const size_t nq = static_cast<size_t>(d.n_heads) * (d.d_nope + d.d_r);
  const size_t part = std::max(static_cast<size_t>(projection_ksplit(d.d_model)) * d_q,
                               static_cast<size_t>(projection_ksplit(d_q)) * nq) * n * sizeof(float);
  return align256(part) + align256(n * d_q * elt);
}

hipError_t launch_query_project(const mla_dims& d, int n_tok, int d_q, const void* x,
                                const void* w_dq, const void* gamma_q, const void* w_uq,
                                const void* w_qr, void* q_nope, void* q_pe, void* ws,
                                hipStream_t s) {
  const size_t elt = d.dtype == MLA_BF16 ? 2 : 4;
  const int C = d.d_model, HD = d.n_heads * d.d_nope, HR = d.n_heads * d.d_r;
  float* y_part = static_cast<float*>(ws);
  const size_t part = query_project_ws_bytes(d, n_tok, d_q) -
                      align256(static_cast<size_t>(n_tok < kProjTok ? n_tok : kProjTok) * d_q * elt);
  char* c_q = static_cast<char*>(ws) + part;  // c_q of the pass, at the activation dtype
  for (int t0 = 0; t0 < n_tok; t0 += kProjTok) {
    const int n = n_tok - t0 < kProjTok ? n_tok - t0 : kProjTok;
    const char* xc = static_cast<const char*>(x) + static_cast<size_t>(t0) * C * elt;
    // query_down and query_norm: c_q = RMSNorm(x · W_DQ) * gamma_q
    hipError_t e = launch_projection_partials(d.dtype, mfma_ok(d, C, d_q, 0), n, C, xc, w_dq, d_q,
                                              nullptr, 0, y_part, s);
    if (e != hipSuccess) return e;
    e = finalize_dt(d.dtype, y_part, projection_ksplit(C), n, d_q, d_q, gamma_q, d.rms_eps,
                    nullptr, c_q, d_q, nullptr, s);
    if (e != hipSuccess) return e;
    // query_up and query_rope: [q_nope | q_pe] = c_q · [W_UQ | W_QR]
    e = launch_projection_partials(d.dtype, mfma_ok(d, d_q, HD, HR), n, d_q, c_q, w_uq, HD, w_qr,
                                   HR, y_part, s);
    if (e != hipSuccess) return e;
    e = finalize_dt(d.dtype, y_part, projection_ksplit(d_q), n, HD + HR, 0, nullptr, 0.f, nullptr,
                    static_cast<char*>(q_nope) + static_cast<size_t>(t0) * HD * elt, HD,
                    static_cast<char*>(q_pe) + static_cast<size_t>(t0) * HR * elt, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

size_t output_project_ws_bytes(const mla_dims& d, int n_tok) {
  const size_t n = static_cast<size_t>(n_tok < kProjTok ? n_tok : kProjTok);
  const int K = d.n_heads * d.d_v;
  return align256(static_cast<size_t>(projection_ksplit(K)) * n * d.d_model * sizeof(float));
}

hipError_t launch_output_project(const mla_dims& d, int n_tok, const void* o, const void* w_o,
                                 const void* b_o, void* y, void* ws, hipStream_t s) {
  const size_t elt = d.dtype == MLA_BF16 ? 2 : 4;
  const int K = d.n_heads * d.d_v, C = d.d_model;
  float* y_part = static_cast<float*>(ws);
  for (int t0 = 0; t0 < n_tok; t0 += kProjTok) {
    const int n = n_tok - t0 < kProjTok ? n_tok - t0 : kProjTok;
    const char* oc = static_cast<const char*>(o) + static_cast<size_t>(t0) * K * elt;
    hipError_t e = launch_projection_partials(d.dtype, mfma_ok(d, K, C, 0), n, K, oc, w_o, C,
                                              nullptr, 0, y_part, s);
    if (e != hipSuccess) return e;
    e = finalize_dt(d.dtype, y_part, projection_ksplit(K), n, C, 0, nullptr, 0.f, b_o,
                    static_cast<char*>(y) + static_cast<size_t>(t0) * C * elt, C, nullptr, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mla
