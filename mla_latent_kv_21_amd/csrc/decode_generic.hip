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
constexpr int kTok = 512;  // most positions scored per pass (one per thread, <= blockDim.x)

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
  // Partials of split k for row r = (b s_q + i) H + h sit at [k * n_rows + r]: one split's rows
  // are contiguous (a workgroup writes one block), a row's splits are n_rows apart.
  void* part_o;  // partial rows, stored at the cache dtype T
  float* part_lse;
  int n_rows;    // batch * s_q * H
  int part_w;    // value width (latent: d_c; GQA: D_v)
};

// One (sequence b, query i, split k, head h) partial: online softmax over the split's positions
// blockDim.x at a time, one position per thread for the scores, one value column per thread
// for the weighted sum. All threads of the block (at most kTok) take part. Scratch: qs[q_w],
// os[part_w], ps[kTok], sl[kTok], red[16] in LDS.
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
  const int pass = static_cast<int>(blockDim.x);
  for (int tt = t0; tt < t1; tt += pass) {
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
    const int nt = min(pass, t1 - tt);
    for (int e = threadIdx.x; e < a.part_w; e += blockDim.x) {
      float acc = os[e] * alpha;
      for (int u = 0; u < nt; ++u) {
        if (sl[u] >= 0) acc += ps[u] * ld(cache, sl[u] * a.row_w + vo + e);
      }
      os[e] = acc;
    }
    __syncthreads();
  }
  const int64_t pidx = static_cast<int64_t>(k) * a.n_rows + qrow;
  const bool any = l > 0.f;
  const float inv = any ? 1.0f / l : 0.f;
  for (int e = threadIdx.x; e < a.part_w; e += blockDim.x)
    st(static_cast<T*>(a.part_o), pidx * a.part_w + e, os[e] * inv);
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

// 16 bytes of T (kVec elements) from p as raw bits; the vector load needs p 16-byte aligned,
// the ragged or unaligned case goes element by element (missing elements are zero).
template <typename T>
__device__ __forceinline__ uint4 load_raw16(const T* p, int n_avail, bool vec_ok) {
  constexpr int kVec = 16 / sizeof(T);
  if (vec_ok && n_avail >= kVec) return *reinterpret_cast<const uint4*>(p);
  union {
    uint4 v;
    T e[kVec];
  } u;
  u.v = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int e = 0; e < kVec; ++e)
    if (e < n_avail) u.e[e] = p[e];
  return u.v;
}

// The kVec elements of T held in 16 raw bytes, as floats.
template <typename T>
__device__ __forceinline__ void widen16(const uint4 raw, float (&v)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  } else {
    v[0] = __uint_as_float(raw.x); v[1] = __uint_as_float(raw.y);
    v[2] = __uint_as_float(raw.z); v[3] = __uint_as_float(raw.w);
  }
}

constexpr int kMaxMergeW = 1024;  // partial row width (d_c or D_v) the merge keeps in LDS
constexpr int kMergeThreads = 512;
constexpr int kMergeU = 8;        // loads in flight per thread per batch (two workgroups per CU)

// One workgroup per (head h, query row m): merges the n_split partials of the row by their
// log-sum-exp (weights 2^(lse_k - max) / sum), then applies the head's group of W_UV
// (out = o_lat · W_UV[:, g(h)]) or, with w_uv NULL (GQA path), stores o_lat itself.
// Every split's partial row is written (an empty split writes zeros), so the partial rows,
// the first W_UV rows and the lse values are all requested at once, before any arithmetic:
//  * thread (column quad cq, split group grp) sums float4 columns of its splits; the groups
//    are added through LDS in group order;
//  * thread (column group cg, row subgroup rs) owns kVec output columns and the W_UV rows
//    j = rs, rs + nrs, ...; the subgroups are added through LDS in subgroup order;
//  * splits the matrix-core kernel flagged are first recomputed exactly (split_head), after
//    which their lse and partial row are read again.
template <typename T>
__global__ __launch_bounds__(kMergeThreads, 4) void merge_kernel(GenericArgs a,
                                                              const int* __restrict__ redo,
                                                              const T* __restrict__ w_uv, int dv,
                                                              T* __restrict__ out,
                                                              float* lse_out) {
  constexpr int kVec = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte load
  extern __shared__ float smem[];
  __shared__ float red[16];
  __shared__ float wts[MLA_MAX_SPLIT];
  __shared__ __attribute__((aligned(16))) float o_s[kMaxMergeW];
  __shared__ float mpart[kMergeThreads * kVec];
  __shared__ float psum[kMergeThreads * kVec];
  __shared__ unsigned long long flagged[kMergeThreads / 64];
  const int n_split = a.n_split, pw = a.part_w, H = a.H;
  const int h = blockIdx.x, m = blockIdx.y;
  const int64_t rh = static_cast<int64_t>(m) * H + h;
  const int tid = threadIdx.x;
  const T* P = static_cast<const T*>(a.part_o) + rh * pw;  // split k at + k * n_rows * pw
  const int64_t kstride = static_cast<int64_t>(a.n_rows) * pw;

  // ---- everything this thread needs first is requested here
  float lk = tid < n_split ? a.part_lse[static_cast<int64_t>(tid) * a.n_rows + rh] : -INFINITY;
  const bool flag = redo != nullptr && tid < n_split &&
                    redo[static_cast<int64_t>(m) * n_split + tid] != 0;
  const int nq = pw / kVec;  // pw % 8 == 0 and pw <= 1024 (checked on the host)
  const int ngrp = min(16, kMergeThreads / nq);
  const int per = cdiv(n_split, ngrp);
  const int cq = tid % nq, grp = tid / nq;
  const bool pthread = grp < ngrp;
  const int k0 = pthread ? grp * per : 0, k1 = pthread ? min(n_split, k0 + per) : 0;
  uint4 v[kMergeU];  // 16 raw bytes of a partial row per split, widened at use
  auto load_parts = [&](int kb) {
#pragma unroll
    for (int u = 0; u < kMergeU; ++u)
      v[u] = kb + u < k1 ? *reinterpret_cast<const uint4*>(P + (kb + u) * kstride + kVec * cq)
                         : make_uint4(0u, 0u, 0u, 0u);
  };
  load_parts(k0);
  const int g = h / (H / a.G);
  const int ncg = cdiv(dv, kVec);  // <= 128 (D_v <= 1024)
  const int nrs = kMergeThreads / ncg;
  const int cg = tid % ncg, rs = tid / ncg;
  const bool wthread = w_uv != nullptr && rs < nrs;
  const int64_t ldw = static_cast<int64_t>(a.G) * dv;
  const T* wc = w_uv + static_cast<int64_t>(g) * dv + cg * kVec;
  const int navail = dv - cg * kVec;
  const bool vec_ok = w_uv != nullptr && (ldw * static_cast<int64_t>(sizeof(T))) % 16 == 0 &&
                      (reinterpret_cast<uintptr_t>(w_uv) & 15u) == 0;
  uint4 wraw[kMergeU];  // 16 raw bytes (kVec elements) of W_UV per row, widened at use
  auto load_w = [&](int jb) {
#pragma unroll
    for (int u = 0; u < kMergeU; ++u) {
      const int j = jb + nrs * u;
      const bool in = wthread && j < pw;
      wraw[u] = load_raw16(wc + static_cast<int64_t>(in ? j : 0) * ldw, in ? navail : 0, vec_ok);
    }
  };
  load_w(rs);

  // ---- splits flagged for exact recomputation (rare): recompute, then read them again
  {
    const unsigned long long bits = __ballot(flag);
    if ((tid & 63) == 0) flagged[tid >> 6] = bits;
    __syncthreads();
    unsigned long long any = 0;
#pragma unroll
    for (int q = 0; q < kMergeThreads / 64; ++q) any |= flagged[q];
    if (any != 0) {
      float* qs = smem;
      float* ro = qs + a.q_w;
      float* ps = ro + pw;
      int64_t* sl = reinterpret_cast<int64_t*>(ps + kTok);
      for (int word = 0; word < kMergeThreads / 64; ++word) {
        unsigned long long left = flagged[word];
        while (left != 0) {
          const int k = word * 64 + __builtin_ctzll(left);
          left &= left - 1;
          split_head<T, false>(a, m / a.s_q, m % a.s_q, k, h, qs, ro, ps, sl, red);
        }
      }
      lk = tid < n_split ? a.part_lse[static_cast<int64_t>(tid) * a.n_rows + rh] : -INFINITY;
      load_parts(k0);
    }
  }

  // ---- weights
  const float mx = block_max(lk, red);
  const float ek = (tid < n_split && mx != -INFINITY) ? exp2f(lk - mx) : 0.f;
  const float sum = block_sum(ek, red);
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  if (tid < n_split) wts[tid] = ek * inv;
  if (tid == 0 && lse_out != nullptr)
    lse_out[rh] = (mx == -INFINITY) ? -INFINITY : (mx + log2f(sum)) * kLn2;
  __syncthreads();

  // ---- o_lat = sum_k w_k o_k into LDS (a split's weight 0 times its finite row adds 0)
  float acc[kVec];
#pragma unroll
  for (int e = 0; e < kVec; ++e) acc[e] = 0.f;
  for (int kb = k0; kb < k1; kb += kMergeU) {
    if (kb != k0) load_parts(kb);
#pragma unroll
    for (int u = 0; u < kMergeU; ++u) {
      const float wk = kb + u < k1 ? wts[kb + u] : 0.f;
      float f[kVec];
      widen16<T>(v[u], f);
#pragma unroll
      for (int e = 0; e < kVec; ++e) acc[e] = fmaf(wk, f[e], acc[e]);
    }
  }
  if (pthread) {
#pragma unroll
    for (int e = 0; e < kVec; ++e) mpart[(grp * nq + cq) * kVec + e] = acc[e];
  }
  __syncthreads();
  if (tid < nq) {
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      float r = mpart[tid * kVec + e];
      for (int q = 1; q < ngrp; ++q) r += mpart[(q * nq + tid) * kVec + e];
      o_s[kVec * tid + e] = r;
    }
  }
  __syncthreads();
  T* orow = out + rh * dv;
  if (w_uv == nullptr) {  // GQA path: the merged rows are the output (pw == dv)
    for (int c = tid; c < dv; c += kMergeThreads) st(orow, c, o_s[c]);
    return;
  }

  // ---- out = o_lat · W_UV[:, g(h)]
  float pacc[kVec];
#pragma unroll
  for (int e = 0; e < kVec; ++e) pacc[e] = 0.f;
  for (int jb = rs; jb < pw; jb += kMergeU * nrs) {
    if (jb != rs) load_w(jb);
#pragma unroll
    for (int u = 0; u < kMergeU; ++u) {
      const int j = jb + nrs * u;
      const float o = j < pw ? o_s[j] : 0.f;
      float wv[kVec];
      widen16<T>(wraw[u], wv);
#pragma unroll
      for (int e = 0; e < kVec; ++e) pacc[e] = fmaf(o, wv[e], pacc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < kVec; ++e) psum[tid * kVec + e] = pacc[e];
  __syncthreads();
  for (int c = tid; c < dv; c += kMergeThreads) {
    const int cgi = c / kVec, e = c - cgi * kVec;
    float r = 0.f;
    for (int q = 0; q < nrs; ++q) r += psum[(q * ncg + cgi) * kVec + e];
    st(orow, c, r);
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
                       void* out, float* lse, hipStream_t s) {
  const int M = batch * a.s_q;
  const size_t lds = redo != nullptr ? split_head_lds(a) : 0;
  hipLaunchKernelGGL(merge_kernel<T>, dim3(a.H, M), dim3(kMergeThreads), lds, s, a, redo,
                     static_cast<const T*>(w_uv), dv, static_cast<T*>(out), lse);
  return hipGetLastError();
}

// Workspace views of one split-K decode.
struct Partials {
  void* o;
  float* lse;
  int* redo;
};

Partials partials_of(void* ws, int batch, int s_q, int heads, int n_split, int width, int elt) {
  const size_t rows = static_cast<size_t>(batch) * s_q * heads * n_split;
  char* base = static_cast<char*>(ws);
  Partials p;
  p.o = base;
  base += (rows * width * elt + 255) / 256 * 256;
  p.lse = reinterpret_cast<float*>(base);
  base += (rows * sizeof(float) + 255) / 256 * 256;
  p.redo = reinterpret_cast<int*>(base);
  return p;
}

GenericArgs latent_args(const mla_dims& d, int batch, int s_q, const void* q_abs, const void* cache,
                        int num_blocks, const int32_t* table, int max_blocks,
                        const int32_t* seq_lens, int n_split, const Partials& p) {
  GenericArgs a{};
  a.q = q_abs; a.cache = cache; a.table = table; a.lens = seq_lens;
  a.num_blocks = num_blocks; a.max_blocks = max_blocks; a.bs = d.block_size;
  a.H = d.n_heads; a.G = d.n_groups; a.s_q = s_q; a.n_split = n_split;
  a.row_w = d.d_c + d.d_r; a.q_w = d.d_c + d.d_r;
  a.d_c = d.d_c; a.d_r = d.d_r; a.D = d.d_nope; a.Dv = d.d_v;
  a.scale_log2 = softmax_scale_of(d) * kLog2e; a.base = d.rope_base;
  a.part_o = p.o; a.part_lse = p.lse; a.part_w = d.d_c; a.n_rows = batch * s_q * d.n_heads;
  return a;
}

bool uses_mfma(const mla_dims& d) {
  return !(d.flags & MLA_FLAG_GENERIC_KERNELS) && mfma_decode_fits(d);
}

}  // namespace

size_t partials_bytes(int batch, int s_q, int heads, int n_split, int width, int elt) {
  const size_t rows = static_cast<size_t>(batch) * s_q * heads * n_split;
  const size_t o = (rows * width * elt + 255) / 256 * 256;
  const size_t l = (rows * sizeof(float) + 255) / 256 * 256;
  const size_t f = (static_cast<size_t>(batch) * s_q * n_split * sizeof(int) + 255) / 256 * 256;
  return o + l + f;
}

hipError_t launch_decode_splitk(const mla_dims& d, int batch, int s_q, const void* q_abs,
                                const void* cache, int num_blocks, const int32_t* table,
                                int max_blocks, const int32_t* seq_lens, int n_split, void* ws,
                                hipStream_t s) {
  const Partials p = partials_of(ws, batch, s_q, d.n_heads, n_split, d.d_c, d.dtype == MLA_BF16 ? 2 : 4);
  if (uses_mfma(d))
    return launch_decode_mfma(d, batch, s_q, q_abs, cache, num_blocks, table, max_blocks,
                              seq_lens, n_split, p.o, p.lse, p.redo, s);
  const GenericArgs a = latent_args(d, batch, s_q, q_abs, cache, num_blocks, table, max_blocks,
                                    seq_lens, n_split, p);
  return d.dtype == MLA_BF16 ? run_generic<bf16, false>(a, batch, s)
                             : run_generic<float, false>(a, batch, s);
}

hipError_t launch_decode_merge(const mla_dims& d, int batch, int s_q, const void* q_abs,
                               const void* cache, int num_blocks, const int32_t* table,
                               int max_blocks, const int32_t* seq_lens, const void* w_uv,
                               int n_split, void* ws, void* out, float* lse, hipStream_t s) {
  const Partials p = partials_of(ws, batch, s_q, d.n_heads, n_split, d.d_c, d.dtype == MLA_BF16 ? 2 : 4);
  const GenericArgs a = latent_args(d, batch, s_q, q_abs, cache, num_blocks, table, max_blocks,
                                    seq_lens, n_split, p);
  // Only the MFMA kernel writes recompute flags; the portable kernel computes every split.
  const int* redo = uses_mfma(d) ? p.redo : nullptr;
  return d.dtype == MLA_BF16 ? run_combine<bf16>(a, redo, batch, d.d_v, w_uv, out, lse, s)
                             : run_combine<float>(a, redo, batch, d.d_v, w_uv, out, lse, s);
}

hipError_t launch_gqa_decode(const mla_dims& d, int batch, int s_q, const void* q_nope,
                             const void* q_pe, const int32_t* q_pos, const void* gqa,
                             int num_blocks, const int32_t* table, int max_blocks,
                             const int32_t* seq_lens, int n_split, void* ws, void* out,
                             float* lse, hipStream_t s) {
  const Partials p = partials_of(ws, batch, s_q, d.n_heads, n_split, d.d_v, d.dtype == MLA_BF16 ? 2 : 4);
  GenericArgs a{};
  a.q = q_nope; a.q_pe = q_pe; a.q_pos = q_pos; a.cache = gqa; a.table = table;
  a.lens = seq_lens; a.num_blocks = num_blocks; a.max_blocks = max_blocks; a.bs = d.block_size;
  a.H = d.n_heads; a.G = d.n_groups; a.s_q = s_q; a.n_split = n_split;
  a.row_w = d.n_groups * (d.d_nope + d.d_v) + d.d_r; a.q_w = d.d_nope + d.d_r;
  a.d_c = d.d_c; a.d_r = d.d_r; a.D = d.d_nope; a.Dv = d.d_v;
  a.scale_log2 = softmax_scale_of(d) * kLog2e; a.base = d.rope_base;
  a.part_o = p.o; a.part_lse = p.lse; a.part_w = d.d_v; a.n_rows = batch * s_q * d.n_heads;
  hipError_t e;
  if (gqa_mfma_fits(d, s_q))
    e = launch_gqa_mfma(d, batch, s_q, q_nope, q_pe, q_pos, gqa, num_blocks, table, max_blocks,
                        seq_lens, n_split, p.o, p.lse, s);
  else
    e = d.dtype == MLA_BF16 ? run_generic<bf16, true>(a, batch, s)
                            : run_generic<float, true>(a, batch, s);
  if (e != hipSuccess) return e;
  return d.dtype == MLA_BF16
             ? run_combine<bf16>(a, nullptr, batch, d.d_v, nullptr, out, lse, s)
             : run_combine<float>(a, nullptr, batch, d.d_v, nullptr, out, lse, s);
}

}  // namespace mla
