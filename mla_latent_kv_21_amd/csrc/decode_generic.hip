// Portable split-K decode kernels (any dims, fp32 or bf16) and the log-sum-exp combine.
//
// Attention per (sequence, query, head) is the textbook softmax of scaled dot products
// (mkdocs.reaper.mx "Le cache clé-valeur", "Le mécanisme d'attention"), taken either in
// latent space over [c || k_r] rows (Smallem article 13, "Ce que DeepSeek fait de plus") or
// over an expanded GQA cache (GQLA summary, "Chemin GQA"). The history of each query is cut
// into n_split chunks reduced independently (online softmax, exp2 of log2-scaled scores);
// the combine kernel merges the chunks by their log-sum-exp and, on the latent path, maps the
// merged latent through the head's group of W_UV once.
#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTok = 256;  // positions scored per pass (one per thread)

struct GenericArgs {
  const void* q;          // latent path: q_abs; GQA path: q_nope
  const void* q_pe;       // GQA path only
  const int32_t* q_pos;   // GQA path only
  const void* cache;
  const int32_t* table;
  const int32_t* lens;
  int num_blocks, max_blocks, bs;
  int H, G, s_q, n_split;
  int row_w;     // elements per cache row
  int q_w;       // query width (latent: d_c + d_r; GQA: D + d_r)
  int d_c, d_r, D, Dv;
  float scale_log2, base;
  float* part_o;
  float* part_lse;
  int part_w;    // value width (latent: d_c; GQA: D_v)
};

// One (sequence b, query i, split k, head h) partial: online softmax over the split's positions
// 256 at a time, one position per thread for the scores, one value column per thread for the
// weighted sum. All threads of the (256-wide) block take part. Scratch: qs[q_w], os[part_w],
// ps[kTok], sl[kTok], red[16] in LDS.
template <typename T, bool kGqa>
__device__ void split_head(const GenericArgs& a, int b, int i, int k, int h, float* qs, float* os,
                           float* ps, int64_t* sl, float* red) {
  const int capacity = a.max_blocks * a.bs;
  const int lim = visible_count(a.lens[b], a.s_q, i, capacity);
  int t0, t1;
  split_range(lim, a.n_split, k, kSplitAlign, &t0, &t1);
  const T* cache = static_cast<const T*>(a.cache);
  const int64_t qrow = (static_cast<int64_t>(b) * a.s_q + i) * a.H + h;
  const int g = h / (a.H / a.G);
  // key segments inside a cache row, and the value segment
  int ko1, kl1, ko2, vo;
  if (kGqa) {
    ko1 = g * a.D; kl1 = a.D; ko2 = a.G * a.D + a.G * a.Dv; vo = a.G * a.D + g * a.Dv;
    const T* qn = static_cast<const T*>(a.q);
    const T* qp = static_cast<const T*>(a.q_pe);
    const int pos = a.q_pos[static_cast<int64_t>(b) * a.s_q + i];
    for (int e = threadIdx.x; e < a.D; e += blockDim.x) qs[e] = ld(qn, qrow * a.D + e);
    for (int j = threadIdx.x; j < a.d_r / 2; j += blockDim.x) {
      float cs, sn;
      rope_cos_sin(pos, j, a.d_r, a.base, &cs, &sn);
      const float x0 = ld(qp, qrow * a.d_r + 2 * j), x1 = ld(qp, qrow * a.d_r + 2 * j + 1);
      qs[a.D + 2 * j] = x0 * cs - x1 * sn;
      qs[a.D + 2 * j + 1] = x0 * sn + x1 * cs;
    }
  } else {
    ko1 = 0; kl1 = a.d_c; ko2 = a.d_c; vo = 0;
    const T* qa = static_cast<const T*>(a.q);
    for (int e = threadIdx.x; e < a.q_w; e += blockDim.x) qs[e] = ld(qa, qrow * a.q_w + e);
  }
  for (int e = threadIdx.x; e < a.part_w; e += blockDim.x) os[e] = 0.f;
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  for (int tt = t0; tt < t1; tt += kTok) {
    const int t = tt + threadIdx.x;
    float s = -INFINITY;
    int64_t slot = -1;
    if (t < t1) slot = cache_slot(a.table, a.max_blocks, a.bs, a.num_blocks, b, t);
    if (slot >= 0) {
      const T* r = cache + slot * a.row_w;
      float acc = 0.f;
      for (int e = 0; e < kl1; ++e) acc += qs[e] * ld(r, ko1 + e);
      for (int e = 0; e < a.d_r; ++e) acc += qs[kl1 + e] * ld(r, ko2 + e);
      s = acc * a.scale_log2;
    }
    sl[threadIdx.x] = slot;
    const float tmax = block_max(s, red);
    const float mn = fmaxf(m, tmax);
    const float p = (s == -INFINITY) ? 0.f : exp2f(s - mn);
    ps[threadIdx.x] = p;
    const float tsum = block_sum(p, red);  // its barriers publish ps and sl
    if (mn == -INFINITY) continue;         // nothing visible in this pass
    const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - mn);
    l = l * alpha + tsum;
    m = mn;
    const int nt = min(kTok, t1 - tt);
    for (int e = threadIdx.x; e < a.part_w; e += blockDim.x) {
      float acc = os[e] * alpha;
      for (int u = 0; u < nt; ++u) {
        if (sl[u] >= 0) acc += ps[u] * ld(cache, sl[u] * a.row_w + vo + e);
      }
      os[e] = acc;
    }
    __syncthreads();
  }
  const int64_t pidx = qrow * a.n_split + k;
  const bool any = l > 0.f;
  const float inv = any ? 1.0f / l : 0.f;
  for (int e = threadIdx.x; e < a.part_w; e += blockDim.x)
    a.part_o[pidx * a.part_w + e] = os[e] * inv;
  if (threadIdx.x == 0) a.part_lse[pidx] = any ? m + log2f(l) : -INFINITY;
  __syncthreads();
}

__host__ __device__ inline size_t split_head_lds(const GenericArgs& a) {
  return (static_cast<size_t>(a.q_w) + a.part_w + kTok) * sizeof(float) + kTok * sizeof(int64_t);
}

template <typename T, bool kGqa>
__global__ __launch_bounds__(256) void decode_generic(GenericArgs a) {
  extern __shared__ float smem[];
  float* qs = smem;
  float* os = qs + a.q_w;
  float* ps = os + a.part_w;
  int64_t* sl = reinterpret_cast<int64_t*>(ps + kTok);
  __shared__ float red[16];
  const int k = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
  for (int h = 0; h < a.H; ++h) split_head<T, kGqa>(a, b, i, k, h, qs, os, ps, sl, red);
}

// Merge of one (sequence, query) row of one head: weights exp2(lse_k - max) / sum over the
// splits, then the weighted sum of the n_split partial vectors, each thread owning two
// columns and keeping eight split loads in flight. With `redo` set, splits the MFMA kernel
// flagged are first recomputed for this head by the portable split routine. Writes the merged
// vector (fp32) to o_lat and the natural-log lse.
__global__ __launch_bounds__(256) void merge_kernel(GenericArgs a, const int* __restrict__ redo,
                                                    int is_bf16, float* __restrict__ o_lat,
                                                    float* lse_out) {
  extern __shared__ float smem[];
  const int n_split = a.n_split, pw = a.part_w, H = a.H;
  float* wts = smem;                     // [n_split]
  __shared__ float red[16];
  const int h = blockIdx.x, m = blockIdx.y;
  const int64_t rh = static_cast<int64_t>(m) * H + h;
  if (redo != nullptr) {
    float* qs = wts + ((n_split + 3) & ~3);
    float* ro = qs + a.q_w;
    float* ps = ro + pw;
    int64_t* sl = reinterpret_cast<int64_t*>(ps + kTok);
    for (int k = 0; k < n_split; ++k) {
      if (redo[static_cast<int64_t>(m) * n_split + k] == 0) continue;
      if (is_bf16)
        split_head<bf16, false>(a, m / a.s_q, m % a.s_q, k, h, qs, ro, ps, sl, red);
      else
        split_head<float, false>(a, m / a.s_q, m % a.s_q, k, h, qs, ro, ps, sl, red);
    }
  }
  const float* L = a.part_lse + rh * n_split;
  float mx = -INFINITY;
  for (int k = threadIdx.x; k < n_split; k += blockDim.x) mx = fmaxf(mx, L[k]);
  mx = block_max(mx, red);
  float sum = 0.f;
  for (int k = threadIdx.x; k < n_split; k += blockDim.x)
    sum += (mx == -INFINITY) ? 0.f : exp2f(L[k] - mx);
  sum = block_sum(sum, red);
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  for (int k = threadIdx.x; k < n_split; k += blockDim.x)
    wts[k] = (mx == -INFINITY) ? 0.f : exp2f(L[k] - mx) * inv;
  if (threadIdx.x == 0 && lse_out != nullptr)
    lse_out[rh] = (mx == -INFINITY) ? -INFINITY : (mx + log2f(sum)) * kLn2;
  __syncthreads();
  const float* P = a.part_o + rh * n_split * pw;
  for (int e = 2 * threadIdx.x; e < pw; e += 2 * blockDim.x) {
    float ax = 0.f, ay = 0.f;
    int k = 0;
    for (; k + 8 <= n_split; k += 8) {
      float2 v[8];
      float wk[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        wk[u] = wts[k + u];
        // empty splits (weight 0) were never written: do not read them
        v[u] = wk[u] != 0.f ? *reinterpret_cast<const float2*>(P + static_cast<int64_t>(k + u) * pw + e)
                            : make_float2(0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) { ax += wk[u] * v[u].x; ay += wk[u] * v[u].y; }
    }
    for (; k < n_split; ++k) {
      const float wk = wts[k];
      if (wk == 0.f) continue;
      const float2 v = *reinterpret_cast<const float2*>(P + static_cast<int64_t>(k) * pw + e);
      ax += wk * v.x;
      ay += wk * v.y;
    }
    *reinterpret_cast<float2*>(o_lat + rh * pw + e) = make_float2(ax, ay);
  }
}

constexpr int kProjRows = 16;
constexpr int kProjCols = 32;

// out[m, h] = o_lat[m, h] · W_UV[:, g(h)] for up to 16 rows m of one head and 32 output
// columns: thread (column c, j-group jg) reduces W_UV rows j = jg*64 .. jg*64+63 for every row
// (each W_UV element is loaded once per workgroup, the loads of a thread all in flight), then
// the 8 j-groups are summed through LDS. w_uv NULL: out = o_lat (GQA path).
template <typename T>
__global__ __launch_bounds__(256) void project_kernel(const float* __restrict__ o_lat, int M,
                                                      int H, int G, int pw, int dv,
                                                      const T* __restrict__ w_uv,
                                                      T* __restrict__ out) {
  extern __shared__ float psm[];
  float* os = psm;                          // [kProjRows][pw]
  float* red = psm + kProjRows * pw;        // [8][kProjRows][kProjCols]
  const int h = blockIdx.x, c0 = blockIdx.y * kProjCols, m0 = blockIdx.z * kProjRows;
  const int g = h / (H / G);
  const int rows = min(kProjRows, M - m0);
  for (int e = threadIdx.x; e < rows * pw; e += blockDim.x) {
    const int r = e / pw, j = e % pw;
    os[e] = o_lat[(static_cast<int64_t>(m0 + r) * H + h) * pw + j];
  }
  __syncthreads();
  const int c = threadIdx.x & (kProjCols - 1), jg = threadIdx.x / kProjCols;  // jg 0..7
  const int v = c0 + c;
  if (w_uv == nullptr) {
    if (jg < rows && v < dv) st(out, (static_cast<int64_t>(m0 + jg) * H + h) * dv + v, os[jg * pw + v]);
    if (jg + 8 < rows && v < dv)
      st(out, (static_cast<int64_t>(m0 + jg + 8) * H + h) * dv + v, os[(jg + 8) * pw + v]);
    return;
  }
  const int64_t ldw = static_cast<int64_t>(G) * dv;
  const T* wc = w_uv + static_cast<int64_t>(g) * dv + (v < dv ? v : 0);
  const int jper = (pw + 7) / 8;
  const int j0 = jg * jper, j1 = min(pw, j0 + jper);
  float acc[kProjRows];
#pragma unroll
  for (int r = 0; r < kProjRows; ++r) acc[r] = 0.f;
  for (int j = j0; j < j1; j += 16) {
    float wv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) wv[u] = (j + u < j1) ? ld(wc, (j + u) * ldw) : 0.f;
#pragma unroll
    for (int r = 0; r < kProjRows; ++r) {
      if (r < rows) {
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (j + u < j1) acc[r] += os[r * pw + j + u] * wv[u];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kProjRows; ++r)
    if (r < rows) red[(jg * kProjRows + r) * kProjCols + c] = acc[r];
  __syncthreads();
  for (int e = threadIdx.x; e < rows * kProjCols; e += blockDim.x) {
    const int r = e / kProjCols, cc = e % kProjCols;
    if (c0 + cc >= dv) continue;
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) sum += red[(q * kProjRows + r) * kProjCols + cc];
    st(out, (static_cast<int64_t>(m0 + r) * H + h) * dv + c0 + cc, sum);
  }
}

template <typename T, bool kGqa>
hipError_t run_generic(const GenericArgs& a, int batch, hipStream_t s) {
  hipLaunchKernelGGL((decode_generic<T, kGqa>), dim3(a.n_split, a.s_q, batch), dim3(256),
                     split_head_lds(a), s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t run_combine(const GenericArgs& a, const int* redo, int batch, int dv, const void* w_uv,
                       float* o_lat, void* out, float* lse, hipStream_t s) {
  const int M = batch * a.s_q;
  size_t lds = ((a.n_split + 3) & ~3) * sizeof(float);
  if (redo != nullptr) lds += split_head_lds(a);
  hipLaunchKernelGGL(merge_kernel, dim3(a.H, M), dim3(256), lds, s, a, redo,
                     static_cast<int>(sizeof(T) == 2), o_lat, lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t plds = (static_cast<size_t>(kProjRows) * a.part_w +
                       8 * kProjRows * kProjCols) * sizeof(float);
  hipLaunchKernelGGL(project_kernel<T>, dim3(a.H, cdiv(dv, kProjCols), cdiv(M, kProjRows)),
                     dim3(256), plds, s, o_lat, M, a.H, a.G, a.part_w, dv,
                     static_cast<const T*>(w_uv), static_cast<T*>(out));
  return hipGetLastError();
}

// Workspace views of one split-K decode.
struct Partials {
  float* o;
  float* lse;
  int* redo;
  float* o_lat;  // merged rows [B, s_q, H, width]
};

Partials partials_of(void* ws, int batch, int s_q, int heads, int n_split, int width) {
  const size_t rows = static_cast<size_t>(batch) * s_q * heads * n_split;
  char* base = static_cast<char*>(ws);
  Partials p;
  p.o = reinterpret_cast<float*>(base);
  base += (rows * width * sizeof(float) + 255) / 256 * 256;
  p.lse = reinterpret_cast<float*>(base);
  base += (rows * sizeof(float) + 255) / 256 * 256;
  p.redo = reinterpret_cast<int*>(base);
  base += (static_cast<size_t>(batch) * s_q * n_split * sizeof(int) + 255) / 256 * 256;
  p.o_lat = reinterpret_cast<float*>(base);
  return p;
}

GenericArgs latent_args(const mla_dims& d, int s_q, const void* q_abs, const void* cache,
                        int num_blocks, const int32_t* table, int max_blocks,
                        const int32_t* seq_lens, int n_split, const Partials& p) {
  GenericArgs a{};
  a.q = q_abs; a.cache = cache; a.table = table; a.lens = seq_lens;
  a.num_blocks = num_blocks; a.max_blocks = max_blocks; a.bs = d.block_size;
  a.H = d.n_heads; a.G = d.n_groups; a.s_q = s_q; a.n_split = n_split;
  a.row_w = d.d_c + d.d_r; a.q_w = d.d_c + d.d_r;
  a.d_c = d.d_c; a.d_r = d.d_r; a.D = d.d_nope; a.Dv = d.d_v;
  a.scale_log2 = softmax_scale_of(d) * kLog2e; a.base = d.rope_base;
  a.part_o = p.o; a.part_lse = p.lse; a.part_w = d.d_c;
  return a;
}

bool uses_mfma(const mla_dims& d) {
  return !(d.flags & MLA_FLAG_GENERIC_KERNELS) && mfma_decode_fits(d);
}

}  // namespace

size_t partials_bytes(int batch, int s_q, int heads, int n_split, int width) {
  const size_t rows = static_cast<size_t>(batch) * s_q * heads * n_split;
  const size_t o = (rows * width * sizeof(float) + 255) / 256 * 256;
  const size_t l = (rows * sizeof(float) + 255) / 256 * 256;
  const size_t f = (static_cast<size_t>(batch) * s_q * n_split * sizeof(int) + 255) / 256 * 256;
  const size_t m = (static_cast<size_t>(batch) * s_q * heads * width * sizeof(float) + 255) / 256 * 256;
  return o + l + f + m;
}

hipError_t launch_decode_splitk(const mla_dims& d, int batch, int s_q, const void* q_abs,
                                const void* cache, int num_blocks, const int32_t* table,
                                int max_blocks, const int32_t* seq_lens, int n_split, void* ws,
                                hipStream_t s) {
  const Partials p = partials_of(ws, batch, s_q, d.n_heads, n_split, d.d_c);
  if (uses_mfma(d))
    return launch_decode_mfma(d, batch, s_q, q_abs, cache, num_blocks, table, max_blocks,
                              seq_lens, n_split, p.o, p.lse, p.redo, s);
  const GenericArgs a = latent_args(d, s_q, q_abs, cache, num_blocks, table, max_blocks,
                                    seq_lens, n_split, p);
  return d.dtype == MLA_BF16 ? run_generic<bf16, false>(a, batch, s)
                             : run_generic<float, false>(a, batch, s);
}

hipError_t launch_decode_merge(const mla_dims& d, int batch, int s_q, const void* q_abs,
                               const void* cache, int num_blocks, const int32_t* table,
                               int max_blocks, const int32_t* seq_lens, const void* w_uv,
                               int n_split, void* ws, void* out, float* lse, hipStream_t s) {
  const Partials p = partials_of(ws, batch, s_q, d.n_heads, n_split, d.d_c);
  const GenericArgs a = latent_args(d, s_q, q_abs, cache, num_blocks, table, max_blocks,
                                    seq_lens, n_split, p);
  // Only the MFMA kernel writes recompute flags; the portable kernel computes every split.
  const int* redo = uses_mfma(d) ? p.redo : nullptr;
  return d.dtype == MLA_BF16 ? run_combine<bf16>(a, redo, batch, d.d_v, w_uv, p.o_lat, out, lse, s)
                             : run_combine<float>(a, redo, batch, d.d_v, w_uv, p.o_lat, out, lse, s);
}

hipError_t launch_gqa_decode(const mla_dims& d, int batch, int s_q, const void* q_nope,
                             const void* q_pe, const int32_t* q_pos, const void* gqa,
                             int num_blocks, const int32_t* table, int max_blocks,
                             const int32_t* seq_lens, int n_split, void* ws, void* out,
                             float* lse, hipStream_t s) {
  const Partials p = partials_of(ws, batch, s_q, d.n_heads, n_split, d.d_v);
  GenericArgs a{};
  a.q = q_nope; a.q_pe = q_pe; a.q_pos = q_pos; a.cache = gqa; a.table = table;
  a.lens = seq_lens; a.num_blocks = num_blocks; a.max_blocks = max_blocks; a.bs = d.block_size;
  a.H = d.n_heads; a.G = d.n_groups; a.s_q = s_q; a.n_split = n_split;
  a.row_w = d.n_groups * (d.d_nope + d.d_v) + d.d_r; a.q_w = d.d_nope + d.d_r;
  a.d_c = d.d_c; a.d_r = d.d_r; a.D = d.d_nope; a.Dv = d.d_v;
  a.scale_log2 = softmax_scale_of(d) * kLog2e; a.base = d.rope_base;
  a.part_o = p.o; a.part_lse = p.lse; a.part_w = d.d_v;
  hipError_t e = d.dtype == MLA_BF16 ? run_generic<bf16, true>(a, batch, s)
                                     : run_generic<float, true>(a, batch, s);
  if (e != hipSuccess) return e;
  return d.dtype == MLA_BF16
             ? run_combine<bf16>(a, nullptr, batch, d.d_v, nullptr, p.o_lat, out, lse, s)
             : run_combine<float>(a, nullptr, batch, d.d_v, nullptr, p.o_lat, out, lse, s);
}

}  // namespace mla
