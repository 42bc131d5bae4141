// The decode layer's projections on either side of the attention path (Smallem article 13,
// "Le code": query_down, query_norm, query_up and query_rope before it, proj after it):
//
//   mla_query_project:  c_q = RMSNorm(x · W_DQ) * gamma_q;  q_nope = c_q · W_UQ;  q_pe = c_q · W_QR
//   mla_output_project: y = o · W_O + b_O
//
// Each product is a split-K projection into fp32 partial sums (fixed K ranges chosen from the
// matrix shape alone, so a token's bits do not depend on the tokens projected with it)
// followed by project_finalize, which sums the partials of one token in a fixed order and
// applies what the step needs: the RMSNorm and gain of query_down, the bias of proj, and the
// split of [W_UQ | W_QR]'s columns into q_nope and q_pe. Tokens go through in passes of at
// most kProjTok, which bounds the workspace.
//
// With a handful of tokens these products are bound by reading the weights once (W_O alone is
// 235 MB at H = 128, D_v = 128, C = 7168), so the bf16 form streams them: project_stream.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"
#include "mfma_util.hpp"

namespace mla {
namespace {

using mfma::bf16x8;
using mfma::f32x16;

constexpr int kSCols = 128;                    // output columns per workgroup (32 per wave)
constexpr int kSRows = 64;                     // K rows per stage
constexpr int kSSlots = 3;                     // stages in the LDS ring
constexpr int kSWBytes = kSRows * kSCols * 2;  // 16 KiB of weights per stage
constexpr int kSXBytes = 32 * kSRows * 2;      // 4 KiB of activations (32 tokens) per stage
constexpr int kSStage = kSWBytes + kSXBytes;
constexpr int kSDma = 5;            // copies per wave per stage (4 of weights, 1 of activations)
constexpr int kSTargetWgs = 512;    // two workgroups per CU
constexpr int kSMinRange = 256;     // shortest K range of one partial sum

// Split-K partials y_part[ks][n][c] = sum over K range ks of x[n][k] * W[k][c] for bf16 x
// [n_tok, K] and W = [W_a | W_b] (row-major [K, n_a] and [K, n_b]). Workgroup (column tile,
// range ks, 32 tokens): four waves of 32 columns; the range streams through a 3-slot LDS ring
// in stages of 64 rows x 128 columns (16 KiB, 256-byte rows) plus the 32 tokens' 64 matching
// activations, copied HBM -> LDS by global_load_lds_dwordx4 two stages ahead. 16-byte pieces
// are XOR-swizzled (weight row r: piece ^ 4 (r % 4); token t: piece ^ (t / 2) % 8) so that
// the operand reads below are free of bank conflicts.
//  * A (tokens x k): 16-byte reads of the activation rows;
//  * B (k x columns): transposing reads (ds_read_b64_tr_b16) of the row-major weight stage.
// Product v_mfma_f32_32x32x16_bf16, four per wave per stage. Rows past n_tok repeat the last
// token (their outputs are not stored). Requires K % 64 == 0, n_a % 128 == 0,
// n_b % 128 == 0, and byte offsets K * max(n_a, n_b) * 2 and n_tok * K * 2 below 2^32.
__global__ __launch_bounds__(256, 2) void project_stream(const char* __restrict__ x,
                                                         const char* __restrict__ w_a,
                                                         const char* __restrict__ w_b,
                                                         int n_tok, int K, int n_a, int n_b,
                                                         int k_range, float* __restrict__ y_part) {
  __shared__ __attribute__((aligned(1024))) char ring[kSSlots][kSStage];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: LDS bases in M0
  const int ncols = n_a + n_b;
  const int c0 = blockIdx.x * kSCols;
  const int ks = blockIdx.y, n0 = blockIdx.z * 32;
  const int kb = ks * k_range;
  const int nt = (min(K, kb + k_range) - kb) / kSRows;
  const bool in_a = c0 < n_a;
  const char* wbase = in_a ? w_a : w_b;
  const int ldw = in_a ? n_a : n_b;
  const int cw = in_a ? c0 : c0 - n_a;

  // copy plan: weight copy i of wave w fills LDS rows 16 w + 4 i + lane / 16, piece lane % 16
  // (which holds the row's piece (lane % 16) ^ 4 (row % 4)); the activation copy of wave w
  // fills tokens 8 w + lane / 8, piece lane % 8 (holding piece (lane % 8) ^ (token / 2) % 8)
  const int wr = lane >> 4, wpc = lane & 15;
  unsigned woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    woff[i] = static_cast<unsigned>((kb + 16 * w + 4 * i + wr) * ldw + cw) * 2u +
              16u * static_cast<unsigned>(wpc ^ (4 * wr));
  const int xt = 8 * w + (lane >> 3), xpc = lane & 7;
  const int xrow = min(n0 + xt, n_tok - 1);
  const unsigned xoff = static_cast<unsigned>(xrow * K + kb) * 2u +
                        16u * static_cast<unsigned>(xpc ^ ((xt >> 1) & 7));
  const unsigned wstep = static_cast<unsigned>(kSRows * ldw) * 2u;
  auto issue = [&](int t, int slot) __attribute__((always_inline)) {
    const unsigned lb = mfma::lds_addr(ring[slot]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      mfma::dma16(wbase, woff[i] + wstep * static_cast<unsigned>(t), lb + 1024u * (4 * w + i));
    mfma::dma16(x, xoff + 2u * kSRows * static_cast<unsigned>(t), lb + kSWBytes + 1024u * w);
  };
  issue(0, 0);
  if (nt > 1) issue(1, 1);

  const int l32 = lane & 31, hi = lane >> 5, G4 = lane >> 4, s16 = lane & 15;
  // B: lane 4 kk + j of 16-lane group G4 reads row 8 (G4 / 2) + kk (+4) of a k-step, columns
  // 32 w + 16 (G4 % 2) + 4 j .. +3, and receives 4 (then 4 more) k of column 32 w + l32
  const int brow = 8 * (G4 >> 1) + (s16 >> 2);
  const int bpc = 4 * w + 2 * (G4 & 1) + ((s16 & 3) >> 1);
  const int boff = brow * (2 * kSCols) + 16 * (bpc ^ (4 * (brow & 3))) + 8 * (s16 & 1);
  f32x16 acc = {};
  for (int t = 0; t < nt; ++t) {
    // stage t has landed once only the next stage's copies may still be in flight
    if (t + 1 < nt)
      mfma::wait_vm<kSDma>();
    else
      mfma::wait_vm<0>();
    __syncthreads();  // every wave's copies of stage t are in; stage t - 1's slot is free
    if (t + 2 < nt) issue(t + 2, (t + 2) % kSSlots);
    const char* sl = ring[t % kSSlots];
#pragma unroll
    for (int s = 0; s < kSRows / 16; ++s) {
      const bf16x8 a = mfma::lds16(sl + kSWBytes + l32 * (2 * kSRows) +
                                   16 * ((2 * s + hi) ^ ((l32 >> 1) & 7)));
      const char* bp = sl + boff + 16 * s * (2 * kSCols);
      const bf16x8 b = mfma::lds_read_tr2(bp, bp + 4 * (2 * kSCols));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
  }
  // D register r holds token 8 (r / 4) + 4 hi + r % 4, column 32 w + l32
  const int col = c0 + 32 * w + l32;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int tok = n0 + 8 * (r >> 2) + 4 * hi + (r & 3);
    if (tok < n_tok) y_part[(static_cast<int64_t>(ks) * n_tok + tok) * ncols + col] = acc[r];
  }
}

bool stream_ok(int K, int n_a, int n_b, int n_tok) {
  const uint64_t ld = static_cast<uint64_t>(std::max(n_a, n_b));
  return K % kSRows == 0 && n_a % kSCols == 0 && n_b % kSCols == 0 && n_a + n_b > 0 &&
         2ull * K * ld < (1ull << 32) && 2ull * n_tok * K < (1ull << 32);
}

// K range of one partial sum of the streaming kernel: about kSTargetWgs workgroups in all,
// from the matrix shape only; never shorter than kSMinRange, so the partial count stays within
// projection_ksplit(K)
int stream_range(int K, int ncols) {
  const int per_col = std::max(1, kSTargetWgs / (ncols / kSCols));
  return std::max(kSMinRange, cdiv(cdiv(K, per_col), kSRows) * kSRows);
}

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

// Partial sums of one pass of n tokens; *n_ksplit receives how many there are.
hipError_t partials(const mla_dims& d, int n, int K, const void* x, const void* w_a, int n_a,
                    const void* w_b, int n_b, float* y_part, int* n_ksplit, hipStream_t s) {
  const bool mfma = mfma_ok(d, K, n_a, n_b);
  if (mfma && stream_ok(K, n_a, n_b, n)) {
    const int ncols = n_a + n_b, kr = stream_range(K, ncols);
    *n_ksplit = cdiv(K, kr);
    hipLaunchKernelGGL(project_stream, dim3(ncols / kSCols, *n_ksplit, cdiv(n, 32)), dim3(256), 0,
                       s, static_cast<const char*>(x), static_cast<const char*>(w_a),
                       static_cast<const char*>(w_b), n, K, n_a, n_b, kr, y_part);
    return hipGetLastError();
  }
  *n_ksplit = projection_ksplit(K);
  return launch_projection_partials(d.dtype, mfma, n, K, x, w_a, n_a, w_b, n_b, y_part, s);
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
    int nk = 0;
    hipError_t e = partials(d, n, C, xc, w_dq, d_q, nullptr, 0, y_part, &nk, s);
    if (e != hipSuccess) return e;
    e = finalize_dt(d.dtype, y_part, nk, n, d_q, d_q, gamma_q, d.rms_eps, nullptr, c_q, d_q,
                    nullptr, s);
    if (e != hipSuccess) return e;
    // query_up and query_rope: [q_nope | q_pe] = c_q · [W_UQ | W_QR]
    e = partials(d, n, d_q, c_q, w_uq, HD, w_qr, HR, y_part, &nk, s);
    if (e != hipSuccess) return e;
    e = finalize_dt(d.dtype, y_part, nk, n, HD + HR, 0, nullptr, 0.f, nullptr,
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
    int nk = 0;
    hipError_t e = partials(d, n, K, oc, w_o, C, nullptr, 0, y_part, &nk, s);
    if (e != hipSuccess) return e;
    e = finalize_dt(d.dtype, y_part, nk, n, C, 0, nullptr, 0.f, b_o,
                    static_cast<char*>(y) + static_cast<size_t>(t0) * C * elt, C, nullptr, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mla
