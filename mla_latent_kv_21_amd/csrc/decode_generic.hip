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
#include "mfma_util.hpp"
#include "plan.hpp"

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
  // Length-balanced plan (in the workspace) or NULL: then split k of row m covers
  // [k chunk, min((k+1) chunk, lim)) and its partial rows sit at [(first[m] + k) H + h].
  const SplitPlan* plan;
  // Latent path with e4m3 rows: one fp32 scale per cache slot (row = bytes x scale), else NULL
  const float* row_scale;
};

// Element e of the cache row at `slot`: of type T, or an e4m3 byte times the row's scale.
template <typename T>
__device__ __forceinline__ float row_elt(const GenericArgs& a, int64_t slot, int e) {
  if (a.row_scale != nullptr) {
    const unsigned char byte =
        static_cast<const unsigned char*>(a.cache)[slot * a.row_w + e];
    return __builtin_amdgcn_cvt_pk_f32_fp8(byte, false)[0] * a.row_scale[slot];
  }
  return ld(static_cast<const T*>(a.cache), slot * a.row_w + e);
}

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
  const int64_t qrow = (static_cast<int64_t>(b) * a.s_q + i) * a.H + h;
  int64_t pidx;
  if (a.plan != nullptr) {
    const int chunk = a.plan->chunk;
    t0 = min(k * chunk, lim);
    t1 = min(t0 + chunk, lim);
    pidx = static_cast<int64_t>(a.plan->first[b * a.s_q + i] + k) * a.H + h;
  } else {
    split_range(lim, a.n_split, k, kSplitAlign, &t0, &t1);
    pidx = static_cast<int64_t>(k) * a.n_rows + qrow;
  }
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
      float acc = 0.f;
      for (int e = 0; e < kl1; ++e) acc += qs[e] * row_elt<T>(a, slot, ko1 + e);
      for (int e = 0; e < a.d_r; ++e) acc += qs[kl1 + e] * row_elt<T>(a, slot, ko2 + e);
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
        if (sl[u] >= 0) acc += ps[u] * row_elt<T>(a, sl[u], vo + e);
      }
      os[e] = acc;
    }
    __syncthreads();
  }
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

// ---------------------------------------------------------------------------------------
// Merge (+ W_UV) for bf16 partials, one workgroup per (head h, block of kRpb query rows: 32,
// or 16, 8, 4 while halving gives the chip more workgroups):
//  * latent path (PW = d_c = 512, D_v = 128): the head's W_UV slice (512 x 128, 128 KiB) is
//    read once for the block's rows instead of once per row, and the projection runs on
//    matrix cores: out^T [128 x 32 rows] = W_UV^T · o_lat^T with v_mfma_f32_32x32x16_bf16,
//    W_UV staged in LDS 256 rows at a time and read with transposing reads, o_lat (bf16 in
//    LDS) read row-wise; wave w < 4 owns output columns 32 w .. 32 w + 31;
//  * GQA path (PW = D_v = 128, no W_UV): the merged rows are the output.
// The partial chunks are requested first, then the splits' lse values, then the W_UV slice.
// Per row the weights 2^(lse_k - max) / sum go to LDS (one wave per row); the merged row is
// o = sum_k w_k o_k. Splits the matrix-core decode flagged are recomputed exactly first
// (split_head), as in merge_kernel.
constexpr int kPjRows = 32, kPjThreads = 512;
constexpr int kPjTargetWgs = 256;  // workgroups that fill the chip (one per CU)
constexpr int kPjDv = 128;
constexpr int kPjORow = 512 * 2 + 16;         // o_lat row in LDS: 1,040 B (rows spread banks)
constexpr int kPjWRow = kPjDv * 2 + 64;       // W_UV row in LDS: 320 B (transposing reads spread)
constexpr int kPjWHalf = 256 * kPjWRow;       // 256 W_UV rows staged at a time (80 KiB)
constexpr int kPjWLoads = 512 * kPjDv * 2 / 16 / kPjThreads;  // 16-byte W loads per thread (16)

template <int PW, bool kProj, bool kPlan, int kRpb>
__global__ __launch_bounds__(kPjThreads) void merge_project_kernel(GenericArgs a,
                                                                const int* __restrict__ redo,
                                                                const uint16_t* __restrict__ w_uv,
                                                                uint16_t* __restrict__ out,
                                                                float* lse_out) {
  static_assert(kRpb == 32 || kRpb == 16 || kRpb == 8 || kRpb == 4, "rows per workgroup");
  static_assert(kPjRows == 32, "rows of the staged o_lat and of the projection's products");
  typedef mfma::bf16x8 bf16x8;
  typedef mfma::f32x16 f32x16;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  static_assert(!kProj || PW == 512, "the projection takes 512-wide latent rows");
  // partial chunks in flight per thread (with W_UV: 8, as 16 and 32 measured slower)
  constexpr int kPjL = kProj ? 8 : 32;
  // a wide batch takes kPjL / S pairs of S <= 8 splits each: at least one, or it never ends
  static_assert(kPjL >= 8, "a wide batch covers at least one pair");
  __shared__ __attribute__((aligned(16))) char wbuf[kProj ? kPjWHalf : 16384];  // W half; scratch
  __shared__ __attribute__((aligned(16))) char obuf[kProj ? kPjRows * kPjORow : 16];
  __shared__ float wts[kPjRows][MLA_MAX_SPLIT];
  __shared__ float red[16];
  __shared__ int n_redo;
  __shared__ int redo_list[256];
  __shared__ int rfirst[kPjRows + 1];  // planned splits: first slot of each row
  const int H = a.H;
  const int h = blockIdx.x, m0 = blockIdx.y * kRpb;
  const int nrv = min(kRpb, a.n_rows / H - m0);  // query rows of this block
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if constexpr (kPlan) {
    if (tid <= nrv) rfirst[tid] = a.plan->first[m0 + tid];
    __syncthreads();
  }
  // splits of row r (uniform: n_split; planned: its own count) and the most of any row here
  auto nk = [&](int r) { return kPlan ? rfirst[r + 1] - rfirst[r] : a.n_split; };
  int n_split = a.n_split;
  if constexpr (kPlan) {
    n_split = 0;
    for (int r = 0; r < nrv; ++r) n_split = max(n_split, nk(r));
  }
  // partial row of split k of row r, and its recompute flag
  auto prow = [&](int r, int k) {
    if constexpr (kPlan) return static_cast<int64_t>(min(rfirst[r] + k, kPlanSlots - 1)) * H + h;
    return static_cast<int64_t>(k) * a.n_rows + static_cast<int64_t>(m0 + r) * H + h;
  };
  auto flag_at = [&](int r, int k) {
    return kPlan ? static_cast<int64_t>(rfirst[r] + k) : static_cast<int64_t>(m0 + r) * a.n_split + k;
  };

  // ---- splits flagged for exact recomputation (rare)
  if (tid == 0) n_redo = 0;
  __syncthreads();
  if (redo != nullptr) {
    for (int e = tid; e < nrv * n_split; e += kPjThreads) {
      const int r = e / n_split, k = e - r * n_split;
      if (k < nk(r) && redo[flag_at(r, k)] != 0) {
        const int slot = atomicAdd(&n_redo, 1);
        if (slot < 256) redo_list[slot] = e;
      }
    }
  }
  __syncthreads();
  if constexpr (kProj) {
    const int nr = n_redo;
    for (int qr = 0; qr < nr; ++qr) {
      int e = -1;
      if (qr < 256) {
        e = redo_list[qr];
      } else {  // more than 256 flags in this block: rescan for the qr-th one
        int seen = 0;
        for (int f = 0; f < nrv * n_split && e < 0; ++f) {
          const int r = f / n_split, k = f - r * n_split;
          if (k < nk(r) && redo[flag_at(r, k)] != 0 && seen++ == qr) e = f;
        }
      }
      const int r = e / n_split, k = e - r * n_split;
      float* qs = reinterpret_cast<float*>(wbuf);
      float* ro = qs + a.q_w;
      float* ps = ro + a.part_w;
      int64_t* sl = reinterpret_cast<int64_t*>(ps + kTok);
      const int mm = m0 + r;
      split_head<bf16, false>(a, mm / a.s_q, mm % a.s_q, k, h, qs, ro, ps, sl, red);
    }
    __syncthreads();
  }

  // ---- this thread's partial chunks, requested before the weights are known. A pair is
  //      (row, 8-column chunk). With few pairs (nq > 1), thread (pair, class q) takes splits
  //      q, q + nq, ...; with few splits (at most 8, rounded up to S = 2^lgS), a thread takes
  //      its pairs t + 512 j in groups of kPjL / S, all their splits at once; otherwise pairs
  //      t + 512 j one after another.
  const int n_pairs = nrv * (PW / 8);
  const int nq = n_pairs >= kPjThreads ? 1 : kPjThreads / n_pairs;
  const bool wide = nq == 1 && n_split <= 8;
  const int lgS = n_split <= 1 ? 0 : n_split <= 2 ? 1 : n_split <= 4 ? 2 : 3;
  int jb = 0;  // wide: first pair group j of the batch
  // byte offsets into the partial rows fit 32 bits (checked at launch): one uniform base
  const char* P = static_cast<const char*>(a.part_o);
  u32x4 v[kPjL];
  auto load_part = [&](int pr, int k) __attribute__((always_inline)) {
    const int r = pr / (PW / 8), c8 = pr - r * (PW / 8);
    const uint32_t off = static_cast<uint32_t>(prow(r, k)) * (PW * 2) + 16u * c8;
    return *reinterpret_cast<const u32x4*>(P + off);
  };
  const int q = nq == 1 ? 0 : tid / n_pairs;
  int pair = nq == 1 ? tid : tid % n_pairs;
  bool live = nq == 1 ? pair < n_pairs : tid < n_pairs * nq;
  int kb = q;
  // one batch: kPjL splits kb + nq u of `pair`, or (wide) split u % S of pair
  // pair + 512 (jb + u / S)
  auto issue = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kPjL; ++u) {
      const int pr = wide ? pair + kPjThreads * (jb + (u >> lgS)) : pair;
      const int k = wide ? u & ((1 << lgS) - 1) : kb + u * nq;
      // past the end: some chunk inside the partials, which gets weight 0
      const int prc = min(pr, n_pairs - 1);
      v[u] = load_part(prc, max(min(k, nk(prc / (PW / 8)) - 1), 0));
    }
  };
  if (live) issue();

  // ---- weights of each row's splits (wave w: rows w, w + 8, ...): every lse value of the
  //      wave's rows is requested before the first reduction waits
  constexpr int kRowsPerWave = kPjRows / (kPjThreads / 64);  // 4
  float lk[kRowsPerWave][MLA_MAX_SPLIT / 64];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int r = w + (kPjThreads / 64) * i;
#pragma unroll
    for (int j = 0; j < MLA_MAX_SPLIT / 64; ++j) {
      const int k = lane + 64 * j;
      lk[i][j] = (r < nrv && k < nk(r)) ? a.part_lse[prow(r, k)] : -INFINITY;
    }
  }
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int r = w + (kPjThreads / 64) * i;
    if (r >= nrv) break;
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < MLA_MAX_SPLIT / 64; ++j) mx = fmaxf(mx, lk[i][j]);
    mx = wave_max(mx);
    float ek[MLA_MAX_SPLIT / 64], sum = 0.f;
#pragma unroll
    for (int j = 0; j < MLA_MAX_SPLIT / 64; ++j) {
      ek[j] = (lane + 64 * j < nk(r) && mx != -INFINITY) ? exp2f(lk[i][j] - mx) : 0.f;
      sum += ek[j];
    }
    sum = wave_sum(sum);
    const float inv = sum > 0.f ? 1.0f / sum : 0.f;
#pragma unroll
    for (int j = 0; j < MLA_MAX_SPLIT / 64; ++j)
      if (lane + 64 * j < n_split) wts[r][lane + 64 * j] = ek[j] * inv;  // 0 past nk(r)
    if (lane == 0 && lse_out != nullptr)
      lse_out[static_cast<int64_t>(m0 + r) * H + h] =
          (mx == -INFINITY) ? -INFINITY : (mx + log2f(sum)) * kLn2;
  }

  // ---- W_UV[:, g D_v .. g D_v + 127], first 256 rows, into registers: thread t holds rows
  //      t / 16 + 32 u, columns 8 (t % 16) .. +7 (the other half is requested after the merge)
  u32x4 wr[kProj ? kPjWLoads / 2 : 1];
  const uint16_t* wsrc = nullptr;
  int64_t ldw = 0;
  if constexpr (kProj) {
    const int g = h / (H / a.G);
    ldw = static_cast<int64_t>(a.G) * kPjDv;
    wsrc = w_uv + static_cast<int64_t>(g) * kPjDv + 8 * (tid & 15) + (tid >> 4) * ldw;
#pragma unroll
    for (int u = 0; u < kPjWLoads / 2; ++u) wr[u] = *reinterpret_cast<const u32x4*>(wsrc + 32 * u * ldw);
  }
  __syncthreads();  // weights published

  // ---- merged rows: o = sum_k w_k o_k (a split's weight 0 times its finite row adds 0)
  float* part_sum = reinterpret_cast<float*>(wbuf);  // [nq][n_pairs][8] when nq > 1
  // a planned row with no split (nothing visible) merges to zero: its chunks were read from a
  // slot that may never have been written
  auto finish = [&](int pr, const float* acc) __attribute__((always_inline)) {
    const int r = pr / (PW / 8), c8 = pr - r * (PW / 8);
    u32x4 o = {mfma::pack_bf16x2(acc[0], acc[1]), mfma::pack_bf16x2(acc[2], acc[3]),
               mfma::pack_bf16x2(acc[4], acc[5]), mfma::pack_bf16x2(acc[6], acc[7])};
    if (kPlan && nk(r) == 0) o = u32x4{0u, 0u, 0u, 0u};
    if constexpr (kProj)
      *reinterpret_cast<u32x4*>(obuf + r * kPjORow + 16 * c8) = o;
    else
      *reinterpret_cast<u32x4*>(out + (static_cast<int64_t>(m0 + r) * H + h) * PW + 8 * c8) = o;
  };
  // chunks past a row's splits are other written chunks of the row, with weight 0
  auto fma8 = [&](float* acc, const u32x4& raw, float wk) __attribute__((always_inline)) {
    float f[8];
    widen16<bf16>(make_uint4(raw[0], raw[1], raw[2], raw[3]), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(wk, f[e], acc[e]);
  };
  if (wide) {
    while (live) {
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
      for (int u = 0; u < kPjL; ++u) {
        const int pr = pair + kPjThreads * (jb + (u >> lgS));
        const int k = u & ((1 << lgS) - 1);
        if (pr < n_pairs) fma8(acc, v[u], k < n_split ? wts[pr / (PW / 8)][k] : 0.f);
        if (k == (1 << lgS) - 1) {  // the pair's splits are summed
          if (pr < n_pairs) finish(pr, acc);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        }
      }
      jb += kPjL >> lgS;
      live = pair + kPjThreads * jb < n_pairs;
      if (live) issue();
    }
  } else {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    while (live) {
      const int r = pair / (PW / 8);
#pragma unroll
      for (int u = 0; u < kPjL; ++u) {
        const int k = kb + u * nq;
        fma8(acc, v[u], k < n_split ? wts[r][k] : 0.f);
      }
      kb += kPjL * nq;
      if (kb >= n_split) {  // this pair's splits are summed
        if (nq == 1) {
          finish(pair, acc);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            part_sum[(static_cast<int64_t>(q) * n_pairs + pair) * 8 + e] = acc[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        kb = q;
        pair += kPjThreads;
        live = nq == 1 && pair < n_pairs;
      }
      if (live) issue();
    }
  }
  if (nq > 1) {
    __syncthreads();
    for (int pr = tid; pr < n_pairs; pr += kPjThreads) {
      float sum8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sum8[e] = part_sum[pr * 8 + e];
      for (int qq = 1; qq < nq; ++qq)
#pragma unroll
        for (int e = 0; e < 8; ++e) sum8[e] += part_sum[(qq * n_pairs + pr) * 8 + e];
      finish(pr, sum8);
    }
  }
  if constexpr (kProj) {
    // ---- out^T = W_UV^T · o_lat^T, two halves of 256 latent rows
    const int l32 = lane & 31, hi = lane >> 5, G4 = lane >> 4, s16 = lane & 15;
    f32x16 pacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) pacc[r] = 0.f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      __syncthreads();  // o_lat is complete / the previous half is consumed
#pragma unroll
      for (int u = 0; u < kPjWLoads / 2; ++u)
        *reinterpret_cast<u32x4*>(wbuf + ((tid >> 4) + 32 * u) * kPjWRow + 16 * (tid & 15)) = wr[u];
      __syncthreads();
      if (half == 0) {  // rows 256 .. 511 arrive while the first half is multiplied
#pragma unroll
        for (int u = 0; u < kPjWLoads / 2; ++u)
          wr[u] = *reinterpret_cast<const u32x4*>(wsrc + (256 + 32 * u) * ldw);
      }
      if (w < kPjDv / 32) {
        // transposing read: 16-lane group G4, source lane 4 kk + j -> W row 16 ks + 8 (G4 / 2)
        // + kk (+4), columns 32 w + 16 (G4 % 2) + 4 j .. +3
        const char* wp = wbuf + (8 * (G4 >> 1) + (s16 >> 2)) * kPjWRow +
                         2 * (32 * w + 16 * (G4 & 1) + 4 * (s16 & 3));
        const char* op = obuf + l32 * kPjORow + 2 * (256 * half + 8 * hi);
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
          const bf16x8 wa = mfma::lds_read_tr2(wp + 16 * ks * kPjWRow, wp + (16 * ks + 4) * kPjWRow);
          const bf16x8 ob = mfma::lds16(op + 32 * ks);
          pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, ob, pacc, 0, 0, 0);
        }
      }
    }
    // register r holds output column 32 w + 8 (r / 4) + 4 hi + r % 4 of row m0 + l32
    if (w < kPjDv / 32 && l32 < nrv) {
      uint16_t* orow = out + (static_cast<int64_t>(m0 + l32) * H + h) * kPjDv + 32 * w + 4 * hi;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<uint2*>(orow + 8 * qd) =
            make_uint2(mfma::pack_bf16x2(pacc[4 * qd], pacc[4 * qd + 1]),
                       mfma::pack_bf16x2(pacc[4 * qd + 2], pacc[4 * qd + 3]));
    }
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
  if constexpr (sizeof(T) == 2) {
    // rows per workgroup of the latent merge: the largest of 32, 16, 8, 4 whose grid fills
    // the chip, else the largest giving the most workgroups (each workgroup reads the head's
    // W_UV slice; splitting a handful of rows that already make one block per head measured
    // slower, but 32 workgroups for 16 rows of 32 heads leave most of the chip idle).
    // A compile-time count: as a run-time one it made the GQA merge twice as slow.
    const bool proj = w_uv != nullptr;
    int rpb = kPjRows;
    if (proj && static_cast<int64_t>(a.H) * cdiv(M, kPjRows) < kPjTargetWgs) {
      rpb = 4;
      for (int r = kPjRows; r > 4; r /= 2)
        if (static_cast<int64_t>(a.H) * cdiv(M, r) >= kPjTargetWgs || cdiv(M, r) == cdiv(M, 4)) {
          rpb = r;
          break;
        }
    }
    const dim3 grid(a.H, cdiv(M, rpb));
    const bool fits32 = a.plan != nullptr ||
                        static_cast<uint64_t>(a.n_split) * a.n_rows * a.part_w * 2 < (1ull << 32);
    if (fits32 && proj && a.part_w == 512 && dv == kPjDv) {
      const uint16_t* wp = static_cast<const uint16_t*>(w_uv);
      uint16_t* op = static_cast<uint16_t*>(out);
#define MLA_MERGE(PLAN_, RPB_)                                                                 \
  hipLaunchKernelGGL((merge_project_kernel<512, true, PLAN_, RPB_>), grid, dim3(kPjThreads), 0, \
                     s, a, redo, wp, op, lse)
      const bool plan = a.plan != nullptr;
      switch (rpb) {
        case 4: if (plan) MLA_MERGE(true, 4); else MLA_MERGE(false, 4); break;
        case 8: if (plan) MLA_MERGE(true, 8); else MLA_MERGE(false, 8); break;
        case 16: if (plan) MLA_MERGE(true, 16); else MLA_MERGE(false, 16); break;
        default: if (plan) MLA_MERGE(true, kPjRows); else MLA_MERGE(false, kPjRows); break;
      }
#undef MLA_MERGE
      return hipGetLastError();
    }
    if (fits32 && a.plan == nullptr && !proj && redo == nullptr && a.part_w == kPjDv &&
        dv == kPjDv) {
      hipLaunchKernelGGL((merge_project_kernel<kPjDv, false, false, kPjRows>), grid,
                         dim3(kPjThreads), 0, s, a, redo, nullptr, static_cast<uint16_t*>(out),
                         lse);
      return hipGetLastError();
    }
  }
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
                        const float* scales, int num_blocks, const int32_t* table, int max_blocks,
                        const int32_t* seq_lens, int n_split, const Partials& p) {
  GenericArgs a{};
  a.row_scale = scales;
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

bool plan_applies(const mla_dims& d, int batch, int s_q) {
  return uses_mfma(d) && d.d_v == kPjDv && batch >= 1 && s_q >= 1 &&
         static_cast<int64_t>(batch) * s_q <= kPlanMaxRows;
}

size_t planned_workspace_bytes(const mla_dims& d) {
  return kPlanBytes + partials_bytes(1, 1, d.n_heads, kPlanSlots, d.d_c, 2);
}

// n_split == 0 here means the length-balanced plan (the caller checked plan_applies): the
// plan sits at the start of the workspace, the partials of the kPlanSlots slots after it.
hipError_t launch_decode_splitk(const mla_dims& d, int batch, int s_q, const void* q_abs,
                                const void* cache, const float* scales, int num_blocks,
                                const int32_t* table, int max_blocks, const int32_t* seq_lens,
                                int n_split, void* ws, hipStream_t s) {
  if (n_split == 0) {
    const Partials p = partials_of(static_cast<char*>(ws) + kPlanBytes, 1, 1, d.n_heads,
                                   kPlanSlots, d.d_c, 2);
    return launch_decode_mfma(d, batch, s_q, q_abs, cache, scales, num_blocks, table, max_blocks,
                              seq_lens, kPlanCap, p.o, p.lse, p.redo,
                              static_cast<SplitPlan*>(ws), nullptr, s);
  }
  const Partials p = partials_of(ws, batch, s_q, d.n_heads, n_split, d.d_c, d.dtype == MLA_BF16 ? 2 : 4);
  if (uses_mfma(d) || scales != nullptr)
    return launch_decode_mfma(d, batch, s_q, q_abs, cache, scales, num_blocks, table, max_blocks,
                              seq_lens, n_split, p.o, p.lse, p.redo, nullptr, nullptr, s);
  const GenericArgs a = latent_args(d, batch, s_q, q_abs, cache, nullptr, num_blocks, table,
                                    max_blocks, seq_lens, n_split, p);
  return d.dtype == MLA_BF16 ? run_generic<bf16, false>(a, batch, s)
                             : run_generic<float, false>(a, batch, s);
}

hipError_t launch_decode_step_splitk(const mla_dims& d, int batch, int s_q, const void* q_abs,
                                     void* cache, int num_blocks, const int32_t* table,
                                     int max_blocks, const int32_t* seq_lens, int n_split,
                                     void* ws, const StepRows& rows, hipStream_t s) {
  // as launch_decode_splitk on the matrix-core kernel, with the new rows formed in the core
  // (e4m3 rows when rows.scale is set: the core reads the scales it writes)
  if (n_split == 0) {
    const Partials p = partials_of(static_cast<char*>(ws) + kPlanBytes, 1, 1, d.n_heads,
                                   kPlanSlots, d.d_c, 2);
    return launch_decode_mfma(d, batch, s_q, q_abs, cache, rows.scale, num_blocks, table,
                              max_blocks, seq_lens, kPlanCap, p.o, p.lse, p.redo,
                              static_cast<SplitPlan*>(ws), &rows, s);
  }
  const Partials p = partials_of(ws, batch, s_q, d.n_heads, n_split, d.d_c, 2);
  return launch_decode_mfma(d, batch, s_q, q_abs, cache, rows.scale, num_blocks, table,
                            max_blocks, seq_lens, n_split, p.o, p.lse, p.redo, nullptr, &rows, s);
}

hipError_t launch_decode_merge(const mla_dims& d, int batch, int s_q, const void* q_abs,
                               const void* cache, const float* scales, int num_blocks,
                               const int32_t* table, int max_blocks, const int32_t* seq_lens,
                               const void* w_uv, int n_split, void* ws, void* out, float* lse,
                               hipStream_t s) {
  if (n_split == 0) {  // length-balanced plan, as in launch_decode_splitk
    const Partials p = partials_of(static_cast<char*>(ws) + kPlanBytes, 1, 1, d.n_heads,
                                   kPlanSlots, d.d_c, 2);
    GenericArgs a = latent_args(d, batch, s_q, q_abs, cache, scales, num_blocks, table,
                                max_blocks, seq_lens, kPlanCap, p);
    a.plan = static_cast<const SplitPlan*>(ws);
    return run_combine<bf16>(a, p.redo, batch, d.d_v, w_uv, out, lse, s);
  }
  const Partials p = partials_of(ws, batch, s_q, d.n_heads, n_split, d.d_c, d.dtype == MLA_BF16 ? 2 : 4);
  const GenericArgs a = latent_args(d, batch, s_q, q_abs, cache, scales, num_blocks, table,
                                    max_blocks, seq_lens, n_split, p);
  // Only the MFMA kernel writes recompute flags; the portable kernel computes every split.
  const int* redo = uses_mfma(d) || scales != nullptr ? p.redo : nullptr;
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
  // many rows per group: four waves share each tile (one split: the kernel writes out and lse)
  const bool shared = prefill_mfma_fits(d, s_q);
  if (shared && n_split == 1)
    return launch_prefill_mfma(d, batch, s_q, q_nope, q_pe, q_pos, gqa, num_blocks, table,
                               max_blocks, seq_lens, 1, out, lse, true, s);
  if (!shared && gqa_mfma_fits(d, s_q) && n_split == 1)
    return launch_gqa_mfma(d, batch, s_q, q_nope, q_pe, q_pos, gqa, num_blocks, table,
                           max_blocks, seq_lens, 1, out, lse, true, s);
  if (shared)
    e = launch_prefill_mfma(d, batch, s_q, q_nope, q_pe, q_pos, gqa, num_blocks, table,
                            max_blocks, seq_lens, n_split, p.o, p.lse, false, s);
  else if (gqa_mfma_fits(d, s_q))
    e = launch_gqa_mfma(d, batch, s_q, q_nope, q_pe, q_pos, gqa, num_blocks, table, max_blocks,
                        seq_lens, n_split, p.o, p.lse, false, s);
  else
    e = d.dtype == MLA_BF16 ? run_generic<bf16, true>(a, batch, s)
                            : run_generic<float, true>(a, batch, s);
  if (e != hipSuccess) return e;
  return d.dtype == MLA_BF16
             ? run_combine<bf16>(a, nullptr, batch, d.d_v, nullptr, out, lse, s)
             : run_combine<float>(a, nullptr, batch, d.d_v, nullptr, out, lse, s);
}

}  // namespace mla
