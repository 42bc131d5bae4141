// Split-K absorbed MLA decode on gfx950 matrix cores: bf16 latent cache with d_c = 512,
// d_r = 64 (1,152-byte rows), H a multiple of 32, fp32 accumulation.
//
// What is computed is the latent-space attention of Smallem article 13, "Ce que DeepSeek fait
// de plus": scores of each absorbed query row against the whole [c || k_r] row (one product
// over the concatenation, "Deux produits ou une concaténation ?"), softmax, and the
// probability-weighted sum of the latents c. Decode is bound by reading the cache
// (GQLA summary, section 1), so the kernel is organised around reading each cache row from
// HBM exactly once and sharing it across all H heads:
//
//  * one workgroup per (split, query, sequence); NW = H/32 waves; wave w owns heads
//    [32w, 32w+32) for the scores and latent columns [512w/NW, 512(w+1)/NW) for the output;
//  * 32-position tiles (36,864 B, always inside one cache block) stream HBM -> LDS with
//    global_load_lds_dwordx4 into a 3-deep ring, so two tiles are in flight while one is
//    used; 16-byte chunks are XOR-swizzled by position so both LDS read patterns below are
//    bank-conflict free;
//  * scores S^T[32 positions x 32 heads] = tile · Q^T with v_mfma_f32_32x32x16_bf16 over the
//    576-wide rows, the wave's absorbed queries held in registers for the whole split;
//  * online softmax in the log2 domain with a lazy rescale (the running max is only raised
//    when a tile exceeds it by more than 2^8, so P <= 256 and the O rescale is rare);
//  * P (bf16) leaves each wave in the exact register layout the next MFMA consumes as its A
//    operand (the position order inside a K-step is permuted consistently on both operands)
//    and is exchanged through LDS; O[H x 512/NW] += P · V with V gathered position-major
//    from the same LDS tile;
//  * each split writes (O / l, m + log2 l) partials; the combine kernel merges splits.
#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kRowElems = 576;            // d_c + d_r
constexpr int kRowBytes = kRowElems * 2;  // 1,152
constexpr int kChunks = kRowBytes / 16;   // 72 sixteen-byte chunks per row
constexpr int kLat = 512;                 // d_c
constexpr int kTileTok = 32;
constexpr int kTileBytes = kTileTok * kRowBytes;  // 36,864
constexpr int kTileChunks = kTileTok * kChunks;   // 2,304
constexpr int kKSteps = kRowElems / 16;           // 36 MFMA K-steps for the scores
constexpr int kRegSteps = 28;                     // query K-steps kept in registers
constexpr int kLdsSteps = kKSteps - kRegSteps;    // the rest (incl. the rotary part) in LDS
constexpr float kHead = 64.0f;                    // P <= 2^kHead, else recompute (log2)
constexpr int kGrp = 4;                           // score K-steps per LDS read group

struct MfmaArgs {
  const uint16_t* q_abs;
  const uint16_t* cache;
  const int32_t* table;
  const int32_t* lens;
  int num_blocks, max_blocks, bs, s_q, n_split;
  float scale_log2;
  float* part_o;
  float* part_lse;
  int* redo;  // [B, s_q, n_split]: 1 where the split must be recomputed
};

typedef __attribute__((address_space(3))) char lds_char_t;

// One 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4): lane i's 16 bytes from
// gbase + off land at LDS byte address lds + 16 i. Issued from asm so that the compiler does
// not order later LDS reads of *other* ring slots behind it; the kernel waits for these
// copies itself (vmcnt) before the barrier that publishes a tile. M0 is restored afterwards.
__device__ __forceinline__ void dma16(const char* gbase, unsigned off, unsigned lds) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(off), "s"(gbase)
      : "memory");
}

__device__ __forceinline__ unsigned lds_addr(const char* p) {
  return static_cast<unsigned>(reinterpret_cast<size_t>((lds_char_t*)p));
}

// Wait until every global -> LDS copy this wave issued has landed.
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

template <int NW>
__device__ __forceinline__ void issue_tile(const MfmaArgs& a, char* buf, int b, int pos0,
                                           int w, int lane_in) {
  // pos0 is a multiple of 32 and bs a multiple of 32, so the tile sits inside one block.
  const int jb = pos0 / a.bs;
  const int id = a.table[static_cast<int64_t>(b) * a.max_blocks + jb];
  const bool ok = id >= 0 && id < a.num_blocks;
  const char* base = reinterpret_cast<const char*>(a.cache) +
                     (static_cast<int64_t>(ok ? id : 0) * a.bs + (pos0 - jb * a.bs)) * kRowBytes;
  // The lane id goes through an empty asm so the per-lane offsets below are recomputed at
  // each issue (a few VALU ops) instead of being hoisted out of the loop into registers.
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
  const unsigned lbase = lds_addr(buf);
  constexpr int kIters = kTileChunks / (NW * 64);
#pragma unroll
  for (int j = 0; j < kIters; ++j) {
    const int p = (j * NW + w) * 64 + lane;  // LDS chunk index this lane fills
    const int t = p / kChunks;
    const int c = (p - t * kChunks) ^ (t & 7);
    dma16(base, static_cast<unsigned>(t * kRowBytes + c * 16), lbase + (j * NW + w) * 64 * 16);
  }
}

// Positions of the tile (relative) that hold valid history: 0 for a bad block id.
__device__ __forceinline__ int tile_valid(const MfmaArgs& a, int b, int pos0, int t1) {
  const int jb = pos0 / a.bs;
  const int id = a.table[static_cast<int64_t>(b) * a.max_blocks + jb];
  const int n = t1 - pos0 < kTileTok ? t1 - pos0 : kTileTok;
  return (id >= 0 && id < a.num_blocks) ? n : 0;
}

template <int NW>
struct Shared {
  bf16x8 p[2][NW][2][64];  // P fragments: [parity][head block][K-step][lane]
  bf16x8 qr[NW][kLdsSteps][64];   // query B operands of the last K-steps
  float inv_l[NW * 32];
  int over[NW];            // a head of the wave outgrew its reference
};

typedef short __attribute__((ext_vector_type(4))) i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane i receives
// element (i % 4) of the 8 bytes addressed by lanes 4k + i/4, for k = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)((lds_char_t*)p));
}

template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mfma_kernel(const uint16_t* __restrict__ q_abs, const uint16_t* __restrict__ cache,
                        const int32_t* __restrict__ table, const int32_t* __restrict__ lens,
                        int num_blocks, int max_blocks, int bs, int s_q, int n_split,
                        float scale_log2, float* __restrict__ part_o,
                        float* __restrict__ part_lse, int* __restrict__ redo) {
  const MfmaArgs a{q_abs, cache, table, lens, num_blocks, max_blocks, bs, s_q, n_split,
                   scale_log2, part_o, part_lse, redo};
  constexpr int H = NW * 32;
  constexpr int kDB = 16 / NW;  // 32-column latent blocks per wave for P · V
  __shared__ __attribute__((aligned(16))) char ring[3][kTileBytes];
  __shared__ Shared<NW> sh;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int k = blockIdx.x, qi = blockIdx.y, b = blockIdx.z;
  const int capacity = a.max_blocks * a.bs;
  const int lim = visible_count(a.lens[b], a.s_q, qi, capacity);
  int t0, t1;
  split_range(lim, a.n_split, k, kSplitAlign, &t0, &t1);
  const int64_t row0 = (static_cast<int64_t>(b) * a.s_q + qi) * H;  // first (b, qi, h) row
  const int64_t split_id = (static_cast<int64_t>(b) * a.s_q + qi) * a.n_split + k;

  if (t0 >= t1) {  // empty split: weight zero in the merge; its o partial is never read
    for (int h = threadIdx.x; h < H; h += blockDim.x)
      a.part_lse[(row0 + h) * a.n_split + k] = -INFINITY;
    if (threadIdx.x == 0) a.redo[split_id] = 0;
    return;
  }

  const int l32 = lane & 31, hi = lane >> 5;

  // Absorbed queries of this wave's 32 heads as MFMA B operands: lane -> head 32w + l32,
  // K-step ks covers row elements [16 ks + 8 hi, +8). The first kRegSteps stay in registers
  // for the whole split; the last ones (the rotary part among them) are parked in LDS to
  // leave registers for the pipeline.
  bf16x8 qf[kRegSteps];
  {
    const char* qp = reinterpret_cast<const char*>(a.q_abs) +
                     (row0 + 32 * w + l32) * kRowBytes + hi * 16;
#pragma unroll
    for (int ks = 0; ks < kRegSteps; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
#pragma unroll
    for (int r = 0; r < kLdsSteps; ++r)
      sh.qr[w][r][lane] = *reinterpret_cast<const bf16x8*>(qp + (kRegSteps + r) * 32);
  }

  // Per-lane LDS byte offsets inside a ring slot; the rest of every swizzled address is a
  // compile-time constant carried in the instruction's offset field.
  //  scores (A operand): position l32, chunk 8g + 2u + hi -> qb[u] + 128 g
  int qb[kGrp];
#pragma unroll
  for (int u = 0; u < kGrp; ++u) qb[u] = l32 * kRowBytes + (((2 * u + hi) ^ (l32 & 7)) << 4);
  //  values (B operand, transposing reads): in 16-lane group G = lane/16, source lane
  //  s = 4 kk + q addresses position 16 k2 + 8 rb + 4 (G/2) + kk and latent columns
  //  (512/NW) w + 32 db + 16 (G%2) + 4 q .. +3 -> vt[db&1] + (16 k2 + 8 rb) * 1152 + (db>>1) * 128
  int vt[2];
  {
    const int G = lane >> 4, s16 = lane & 15, kk = s16 >> 2, q = s16 & 3;
    const int tokA = 4 * (G >> 1) + kk;  // position within the 16-position step, < 8
#pragma unroll
    for (int dp = 0; dp < 2; ++dp)
      vt[dp] = tokA * kRowBytes + (((4 * dp + 2 * (G & 1) + (q >> 1)) ^ tokA) << 4) +
               8 * (q & 1) + (8 / NW) * w * 128;
  }

  f32x16 o[NW * kDB];
#pragma unroll
  for (int j = 0; j < NW * kDB; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[j][r] = 0.f;
  float m_ref = -INFINITY;  // reference max (log2 units) of head 32w + l32
  float l_part = 0.f;       // this lane's share of the softmax denominator
  bool over = false;
  const int ntiles = cdiv(t1 - t0, kTileTok);

  // ---- scores S^T[position][head] of one tile over the 576-wide rows; fragments are read
  // one group ahead of their MFMAs.
  auto scores = [&](const char* cur) __attribute__((always_inline)) -> f32x16 {
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
    bf16x8 cf[kGrp], nf[kGrp];
#pragma unroll
    for (int u = 0; u < kGrp; ++u) cf[u] = *reinterpret_cast<const bf16x8*>(cur + qb[u]);
#pragma unroll
    for (int g = 0; g < kKSteps / kGrp; ++g) {
      if (g + 1 < kKSteps / kGrp) {
#pragma unroll
        for (int u = 0; u < kGrp; ++u)
          nf[u] = *reinterpret_cast<const bf16x8*>(cur + qb[u] + 128 * (g + 1));
      }
#pragma unroll
      for (int u = 0; u < kGrp; ++u) {
        const int ks = g * kGrp + u;
        const bf16x8 qv = ks < kRegSteps ? qf[ks < kRegSteps ? ks : 0] : sh.qr[w][ks - kRegSteps][lane];
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cf[u], qv, sc, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kGrp; ++u) cf[u] = nf[u];
    }
    return sc;
  };

  // ---- softmax numerators of one tile against the head's fixed reference m_ref (log2
  // units): the first finite tile max. A tile exceeding it by more than kHead marks the split
  // for exact recomputation instead of rescaling O, so O is only ever touched by MFMAs. The
  // numerators are left in P's LDS slot `par` as the next MFMA's A operand.
  auto softmax = [&](f32x16 sc, int nvalid, int par) __attribute__((always_inline)) {
    if (nvalid < kTileTok) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + 4 * hi + (r & 3) >= nvalid) sc[r] = -INFINITY;
    }
    float mr = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mr = fmaxf(mr, sc[r]);
    mr = fmaxf(mr, __shfl_xor(mr, 32, 64));
    const float mt = mr * a.scale_log2;
    if (m_ref == -INFINITY) m_ref = mt;  // nothing accumulated yet for this head
    over = over || (mt > m_ref + kHead);
    const float neg = m_ref == -INFINITY ? 0.f : -m_ref;  // all-masked so far: p = 0 anyway
    float psum = 0.f;
    bf16x8 pf[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2f(fmaf(sc[r], a.scale_log2, neg));
      psum += p;
      pf[r >> 3][r & 7] = static_cast<__bf16>(p);
    }
    l_part += psum;
    sh.p[par][w][0][lane] = pf[0];
    sh.p[par][w][1][lane] = pf[1];
  };

  // ---- O[heads x wave's latent columns] += P · V for one tile, 16 positions per K-step
  // Rows of a partial tile past the history are zeroed in LDS before its P · V (their scores
  // are masked, but 0 x NaN would still poison O).
  auto zero_tail = [&](char* cur, int nvalid) __attribute__((always_inline)) {
    const int from = nvalid * kChunks, to = kTileChunks;
    for (int c = from + static_cast<int>(threadIdx.x); c < to; c += NW * 64)
      *reinterpret_cast<uint4*>(cur + 16 * c) = make_uint4(0u, 0u, 0u, 0u);
  };

  auto pv = [&](const char* cur, int par) __attribute__((always_inline)) {
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      bf16x8 pa[NW];
#pragma unroll
      for (int hb = 0; hb < NW; ++hb) pa[hb] = sh.p[par][hb][k2][lane];
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const char* vp = cur + vt[db & 1] + 16 * k2 * kRowBytes + (db >> 1) * 128;
        const i16x4 v0 = lds_read_tr(vp);
        const i16x4 v1 = lds_read_tr(vp + 8 * kRowBytes);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int hb = 0; hb < NW; ++hb)
          o[hb * kDB + db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[hb], vf, o[hb * kDB + db],
                                                                     0, 0, 0);
      }
    }
  };

  // ---- pipeline: tiles t and t+1 sit in the ring while tile t+2 streams in; the scores and
  // softmax of tile t+1 are formed before P · V of tile t so their VALU work can overlap it.
  issue_tile<NW>(a, ring[0], b, t0, w, lane);
  if (ntiles > 1) issue_tile<NW>(a, ring[1], b, t0 + kTileTok, w, lane);
  wait_dma();
  __syncthreads();
  {
    const int nv0 = tile_valid(a, b, t0, t1);
    softmax(scores(ring[0]), nv0, 0);
    if (nv0 < kTileTok) zero_tail(ring[0], nv0);
  }

  for (int t = 0; t < ntiles; ++t) {
    const int slot = t % 3;
    const int nslot = slot == 2 ? 0 : slot + 1;
    const int pos0 = t0 + t * kTileTok;
    // P(t) and the zeroed tail of tile t become visible to every wave, tile t+1 has landed,
    // the slot of tile t-1 is free.
    wait_dma();
    __syncthreads();
    if (t + 2 < ntiles) issue_tile<NW>(a, ring[slot == 0 ? 2 : slot - 1], b, pos0 + 2 * kTileTok, w, lane);
    // On the last tile the next slot holds stale data; with no valid position the softmax
    // below masks every score and leaves m_ref, l and the flag unchanged.
    const int nv_next = t + 1 < ntiles ? tile_valid(a, b, pos0 + kTileTok, t1) : 0;
    const f32x16 sc = scores(ring[nslot]);
    pv(ring[slot], t & 1);
    softmax(sc, nv_next, (t + 1) & 1);
    // zeroed before the next barrier, which also orders it after every wave's scores
    if (t + 1 < ntiles && nv_next < kTileTok) zero_tail(ring[nslot], nv_next);
  }

  // ---- partials: o / l and m_ref + log2(l) per head, plus the recompute flag
  const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
  const bool wover = __builtin_amdgcn_ballot_w64(over) != 0;
  if (lane == 0) sh.over[w] = wover ? 1 : 0;
  if (lane < 32) {
    const int h = 32 * w + lane;
    sh.inv_l[h] = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    a.part_lse[(row0 + h) * a.n_split + k] = l_tot > 0.f ? m_ref + log2f(l_tot) : -INFINITY;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int any = 0;
#pragma unroll
    for (int j = 0; j < NW; ++j) any |= sh.over[j];
    a.redo[split_id] = any;
  }
#pragma unroll
  for (int hb = 0; hb < NW; ++hb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int h = 32 * hb + 8 * (r >> 2) + 4 * hi + (r & 3);
      const float il = sh.inv_l[h];
      float* dst = a.part_o + ((row0 + h) * a.n_split + k) * kLat + (kLat / NW) * w + l32;
#pragma unroll
      for (int db = 0; db < kDB; ++db) dst[32 * db] = o[hb * kDB + db][r] * il;
    }
  }
}

}  // namespace

bool mfma_decode_fits(const mla_dims& d) {
  return d.dtype == MLA_BF16 && d.d_c == 512 && d.d_r == 64 && d.block_size % 32 == 0 &&
         (d.n_heads == 32 || d.n_heads == 64 || d.n_heads == 128);
}

hipError_t launch_decode_mfma(const mla_dims& d, int batch, int s_q, const void* q_abs,
                              const void* cache, int num_blocks, const int32_t* table,
                              int max_blocks, const int32_t* seq_lens, int n_split,
                              float* part_o, float* part_lse, int* redo, hipStream_t s) {
  MfmaArgs a;
  a.q_abs = static_cast<const uint16_t*>(q_abs);
  a.cache = static_cast<const uint16_t*>(cache);
  a.table = table;
  a.lens = seq_lens;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks;
  a.bs = d.block_size;
  a.s_q = s_q;
  a.n_split = n_split;
  a.scale_log2 = softmax_scale_of(d) * 1.4426950408889634f;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.redo = redo;
  const dim3 grid(n_split, s_q, batch);
#define MLA_LAUNCH(NW_)                                                                        \
  hipLaunchKernelGGL(decode_mfma_kernel<NW_>, grid, dim3(64 * NW_), 0, s, a.q_abs, a.cache,     \
                     a.table, a.lens, a.num_blocks, a.max_blocks, a.bs, a.s_q, a.n_split,       \
                     a.scale_log2, a.part_o, a.part_lse, a.redo)
  switch (d.n_heads) {
    case 128: MLA_LAUNCH(4); break;
    case 64: MLA_LAUNCH(2); break;
    default: MLA_LAUNCH(1); break;
  }
#undef MLA_LAUNCH
  return hipGetLastError();
}

}  // namespace mla
