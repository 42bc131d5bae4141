// Split-K absorbed MLA decode on gfx950 matrix cores: bf16 latent cache with d_c = 512,
// d_r = 64 (1,152-byte rows), H in {32, 64, 128}, fp32 accumulation.
//
// What is computed is the latent-space attention of Smallem article 13, "Ce que DeepSeek fait
// de plus": scores of each absorbed query row against the whole [c || k_r] row (one product
// over the concatenation, "Deux produits ou une concaténation ?"), softmax, and the
// probability-weighted sum of the latents c. Decode is bound by reading the cache
// (GQLA summary, section 1), so the kernel is organised around reading each cache row from
// HBM exactly once and sharing it across all H heads:
//
//  * one workgroup per (split, query, sequence); NW = H/32 waves; wave w owns heads
//    [32w, 32w+32) for the scores and latent columns [512w/NW, 512(w+1)/NW) of all heads for
//    the output;
//  * 32-position tiles (36,864 B, always inside one cache block) stream HBM -> LDS with
//    global_load_lds_dwordx4 into a 4-slot ring, two tiles in flight; 16-byte
//    chunks are XOR-swizzled by position so every LDS read pattern below is free of bank
//    conflicts;
//  * scores S^T[32 positions x 32 heads] = tile · Q^T with v_mfma_f32_32x32x16_bf16 over the
//    576-wide rows, the wave's absorbed queries held in registers for the whole split;
//  * softmax against a fixed per-head reference (the first finite tile max, log2 domain):
//    O is never rescaled; a tile exceeding the reference by more than 2^64 flags the split,
//    which the merge kernel then recomputes exactly;
//  * P (bf16) leaves each wave in the register layout the P · V product consumes as its A
//    operand (the position order inside a K-step is permuted identically on both operands)
//    and is exchanged through LDS; O[H x 512/NW] += P · V with V read by transposing LDS
//    reads from the same tile;
//  * the loop body is scheduled by hand: the scores of tile t+1 run with their LDS reads
//    several steps ahead, then P · V of tile t runs with the softmax of tile t+1 spread
//    between its products, so the matrix cores are fed while the VALU and LDS work;
//  * each split writes (O / l as bf16, m + log2 l) partials; the merge kernel combines them.
#include "common.hpp"
#include "launch.hpp"
#include "plan.hpp"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef short __attribute__((ext_vector_type(4))) i16x4;

constexpr int kRowElems = 576;            // d_c + d_r
constexpr int kRowBytes = kRowElems * 2;  // 1,152
constexpr int kChunks = kRowBytes / 16;   // 72 sixteen-byte chunks per row
constexpr int kLat = 512;                 // d_c
constexpr int kTileTok = 32;
constexpr int kTileBytes = kTileTok * kRowBytes;  // 36,864
constexpr int kTileChunks = kTileTok * kChunks;   // 2,304
constexpr int kKSteps = kRowElems / 16;           // 36 MFMA K-steps for the scores
constexpr float kHead = 64.0f;                    // P <= 2^kHead, else recompute (log2)
constexpr int kPre = 10;                          // score fragments read ahead of their MFMA
constexpr int kVPre = 2;                          // P · V steps whose V fragments are in flight
constexpr int kSlots = 4;                         // ring slots: two tiles in flight

typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// Physical 16-byte chunk of logical chunk c in tile row t is c ^ swz(t). swz is a linear map
// of the row's low four bits into three bits (a row's 72 chunks stay in their groups of 8).
// It is chosen so that the score reads (16 bytes per lane, 32 rows x one chunk pair) and the
// transposing value reads (8 bytes per lane, 4 rows x 2 chunks per 16 lanes) hit distinct
// banks within every 128- and 256-byte LDS beat.
__host__ __device__ constexpr int swz(int t) {
  return ((t & 1) ? 3 : 0) ^ ((t & 2) ? 4 : 0) ^ ((t & 4) ? 2 : 0) ^ ((t & 8) ? 1 : 0);
}

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

// s_waitcnt immediate that waits for vmcnt <= n only (expcnt and lgkmcnt at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait until at most `later` global -> LDS copies issued by this wave are still in flight:
// copies complete in issue order, so everything issued before them has landed.
template <int kLater>
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLater)); }

// O += A · B with O held in accumulation registers (AGPRs). The score products use the
// compiler's MFMA in its VGPR form (this file is built with MFMA results in VGPRs), so that
// O (256 AGPRs) and the score accumulator never compete for one register file. The compiler
// does not track this instruction's hazards: the leading s_nop covers a VALU write of A or B
// just before it (two wait states); O is only ever written by this instruction, and is read
// only after the explicit wait that follows the main loop.
__device__ __forceinline__ void mfma_o(f32x16& o, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(b));
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane i receives
// element (i % 4) of the 8 bytes addressed by lanes 4k + i/4, for k = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)((lds_char_t*)p));
}

__device__ __forceinline__ bf16x8 lds16(const char* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// two floats as a bf16 pair (round to nearest even), low element first
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(unsigned, v);
}

// max over the lane pair (lane, lane ^ 32), without going through LDS
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int NW>
struct Shared {
  bf16x8 p[2][NW][2][64];         // P fragments: [parity][head block][K-step][lane]
};
// After the loop the ring is free and holds the per-head 1/l and the waves' flags.
template <int NW>
struct Tail {
  float inv_l[NW * 32];
  int over[NW];                   // a head of the wave outgrew its reference
};

struct SoftState {
  float m1, m2, m3, m4, m5, m6, mr, neg, psum;
  bf16x8 pf[2];
};

template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mfma_kernel(const uint16_t* __restrict__ q_abs, const uint16_t* __restrict__ cache,
                        const int32_t* __restrict__ table, const int32_t* __restrict__ lens,
                        int num_blocks, int max_blocks, int bs, int s_q, int n_split,
                        float scale_log2, uint16_t* __restrict__ part_o,
                        float* __restrict__ part_lse, int* __restrict__ redo, int batch,
                        SplitPlan* __restrict__ plan_out) {
  constexpr int H = NW * 32;
  constexpr int kDB = 16 / NW;                      // 32-column latent blocks per wave
  constexpr int kPV = 2 * kDB * NW;                 // P · V products per tile (32)
  constexpr int kDma = kTileChunks / (NW * 64);     // copies per wave per tile
  static_assert(kDma <= kKSteps, "copies are spread over the score K-steps");
  __shared__ __attribute__((aligned(16))) char ring[kSlots][kTileBytes];
  __shared__ Shared<NW> sh;
  static_assert(sizeof(ring) + sizeof(Shared<NW>) <= 160 * 1024, "LDS");

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int capacity = max_blocks * bs;
  int k, qi, b, t0, t1;
  int64_t split_id, prow0;
  if (plan_out == nullptr) {
    // uniform split: workgroup (k, qi, b); partial rows of split k at [k * n_rows + row]
    k = blockIdx.x; qi = blockIdx.y; b = blockIdx.z;
    const int lim = visible_count(lens[b], s_q, qi, capacity);
    split_range(lim, n_split, k, kSplitAlign, &t0, &t1);
    const int64_t m = static_cast<int64_t>(b) * s_q + qi;
    split_id = m * n_split + k;
    prow0 = k * (static_cast<int64_t>(batch) * s_q * H) + m * H;
  } else {
    // length-balanced plan: workgroup = split slot; partial rows of slot s at [s H + h]
    SplitPlan* pl = reinterpret_cast<SplitPlan*>(ring[0]);
    int* row_of = reinterpret_cast<int*>(ring[1]);
    const int slot = blockIdx.x;
    make_plan(lens, batch, s_q, capacity, slot, pl, row_of);
    if (slot >= pl->total) return;
    const int rows = batch * s_q;
    if (slot == 0) {
      int* dst = reinterpret_cast<int*>(plan_out);
      const int* src = reinterpret_cast<const int*>(pl);
      for (int e = threadIdx.x; e < 2 + rows + 1; e += blockDim.x) dst[e] = src[e];
    }
    const int m = __builtin_amdgcn_readfirstlane(row_of[0]);
    const int chunk = __builtin_amdgcn_readfirstlane(pl->chunk);
    b = m / s_q; qi = m - b * s_q;
    k = slot - __builtin_amdgcn_readfirstlane(pl->first[m]);
    const int lim = __builtin_amdgcn_readfirstlane(row_of[1]);
    t0 = k * chunk;
    t1 = min(t0 + chunk, lim);
    split_id = slot;
    prow0 = static_cast<int64_t>(slot) * H;
    __syncthreads();  // the plan is read before the ring takes tiles
  }
  const int64_t row0 = (static_cast<int64_t>(b) * s_q + qi) * H;  // first (b, qi, h) query row

  if (t0 >= t1) {  // empty split: lse -inf (weight zero in the merge) and a zero partial row
    for (int h = threadIdx.x; h < H; h += blockDim.x) part_lse[prow0 + h] = -INFINITY;
    for (int e = threadIdx.x; e < H * (kLat / 8); e += blockDim.x)
      *reinterpret_cast<uint4*>(part_o + prow0 * kLat + 8 * e) = make_uint4(0u, 0u, 0u, 0u);
    if (threadIdx.x == 0) redo[split_id] = 0;
    return;
  }

  const int l32 = lane & 31, hi = lane >> 5;

  // Absorbed queries of this wave's 32 heads as MFMA B operands, in registers for the whole
  // split: lane -> head 32w + l32, K-step ks covers row elements [16 ks + 8 hi, +8). Loaded
  // after the first tile's copies are issued.
  bf16x8 qf[kKSteps];

  // Per-lane byte offsets; the rest of every swizzled address is a compile-time constant.
  //  copies: LDS chunk p = (j NW + w) 64 + lane of a slot holds row p / 72, physical chunk
  //  p % 72, i.e. logical chunk (p % 72) ^ swz(row) of the cache rows.
  unsigned doff[kDma];
#pragma unroll
  for (int j = 0; j < kDma; ++j) {
    const int p = (j * NW + w) * 64 + lane;
    const int t = p / kChunks;
    const int c = p - t * kChunks;
    doff[j] = static_cast<unsigned>(t * kRowBytes + ((c ^ swz(t)) << 4));
  }
  //  scores (A operand): position l32, K-step ks = 4 g + u reads logical chunk 2 ks + hi
  //  = 8 g + 2 u + hi -> qb[u] + 128 g
  int qb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) qb[u] = l32 * kRowBytes + (((2 * u + hi) ^ swz(l32)) << 4);
  //  values (B operand, transposing reads): in 16-lane group G = lane/16, source lane
  //  s = 4 kk + q addresses position 16 k2 + 8 rb + 4 (G/2) + kk and latent columns
  //  (512/NW) w + 32 db + 16 (G%2) + 4 q .. +3 -> vt[db&1][rb] + 16 k2 * 1152 + (db>>1) * 128
  int vt[2][2];
  {
    const int G = lane >> 4, s16 = lane & 15, kk = s16 >> 2, q = s16 & 3;
    const int tokA = 4 * (G >> 1) + kk;
#pragma unroll
    for (int dp = 0; dp < 2; ++dp)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int t = 8 * rb + tokA;
        vt[dp][rb] = t * kRowBytes + (((4 * dp + 2 * (G & 1) + (q >> 1)) ^ swz(t)) << 4) +
                     8 * (q & 1) + (8 / NW) * w * 128;
      }
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

  // Block ids of the split, one per lane (lane i: block jbase + i of the sequence), so a
  // tile's id is a v_readlane instead of a scalar load waited on in the loop; reloaded when
  // the split moves past 64 blocks (tiles are visited in increasing order).
  // The load is issued from asm with its own wait: a compiler-visible vector load in the loop
  // would make the compiler wait for every copy in flight before each use of `ids`.
  int jbase = t0 / bs;
  auto load_ids = [&]() {
    const int jj = jbase + lane;
    const int32_t* src = table + static_cast<int64_t>(b) * max_blocks + (jj < max_blocks ? jj : 0);
    int v;
    asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(src) : "memory");
    return jj < max_blocks ? v : -1;
  };
  int ids = load_ids();
  // Cache address of the tile at pos0 (a multiple of 32 inside one block) and its number of
  // valid positions (0 for a bad block id, whose rows are then never used).
  const int64_t blk_bytes = static_cast<int64_t>(bs) * kRowBytes;
  // jb = pos0 / bs and off = pos0 - jb * bs are passed in (the loop tracks them incrementally)
  auto tile_src_at = [&](int pos0, int jb, int off, int* nvalid) -> const char* {
    if (jb - jbase >= 64) {
      jbase = jb;
      ids = load_ids();
    }
    const int id = __builtin_amdgcn_readlane(ids, jb - jbase);
    const bool ok = id >= 0 && id < num_blocks;
    const int n = t1 - pos0 < kTileTok ? t1 - pos0 : kTileTok;
    *nvalid = ok ? n : 0;
    return reinterpret_cast<const char*>(cache) + (ok ? id : 0) * blk_bytes + off * kRowBytes;
  };
  auto tile_src = [&](int pos0, int* nvalid) -> const char* {
    const int jb = pos0 / bs;
    return tile_src_at(pos0, jb, pos0 - jb * bs, nvalid);
  };
  auto issue_tile = [&](const char* src, char* slot) __attribute__((always_inline)) {
    const unsigned lbase = lds_addr(slot) + w * 64 * 16;
#pragma unroll
    for (int j = 0; j < kDma; ++j) dma16(src, doff[j], lbase + j * NW * 64 * 16);
  };
  // Copy j of a tile issued from inside the score loop: the copies of the four waves then
  // spread over the score phase instead of queueing at the vector-memory unit together.
  auto issue_part = [&](const char* src, unsigned lbase, int j) __attribute__((always_inline)) {
    if (src != nullptr) dma16(src, doff[j], lbase + j * NW * 64 * 16);
  };

  // ---- scores S^T[position][head] of one tile over the 576-wide rows, each fragment read
  // kPre products ahead of its MFMA.
  auto scores = [&](const char* cur, const char* dsrc, unsigned dlds)
                    __attribute__((always_inline)) -> f32x16 {
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
    bf16x8 af[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i) af[i] = lds16(cur + qb[i & 3] + 128 * (i >> 2));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const bf16x8 acur = af[ks % kPre];
      const int nx = ks + kPre;
      if (nx < kKSteps) af[ks % kPre] = lds16(cur + qb[nx & 3] + 128 * (nx >> 2));
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(acur, qf[ks], sc, 0, 0, 0);
      // copies spread evenly over the K-steps (kDma <= kKSteps)
      if ((ks * kDma) / kKSteps != ((ks + 1) * kDma) / kKSteps)
        issue_part(dsrc, dlds, (ks * kDma) / kKSteps);
      __builtin_amdgcn_sched_barrier(0);
    }
    return sc;
  };

  // ---- softmax numerators of one tile against the head's fixed reference m_ref (log2
  // units): the first finite tile max. A tile exceeding it by more than kHead marks the split
  // for exact recomputation instead of rescaling O, so O is only ever touched by MFMAs. The
  // numerators are left in P's LDS slot `par` as the A operand of the next P · V.
  // Split in pieces (compile-time numbers) so the unmasked case can be spread between the
  // P · V products.
  constexpr int kSoftPieces = 26;
  auto soft_piece = [&](int piece, f32x16& sc, SoftState& s, int par)
                        __attribute__((always_inline)) {
    if (piece == 0) {
      s.m1 = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
      s.m2 = fmaxf(fmaxf(sc[3], sc[4]), sc[5]);
      s.m3 = fmaxf(fmaxf(sc[6], sc[7]), sc[8]);
    } else if (piece == 1) {
      s.m4 = fmaxf(fmaxf(sc[9], sc[10]), sc[11]);
      s.m5 = fmaxf(fmaxf(sc[12], sc[13]), sc[14]);
      s.m6 = fmaxf(fmaxf(sc[15], s.m1), s.m2);
    } else if (piece == 2) {
      s.mr = fmaxf(fmaxf(fmaxf(s.m3, s.m4), s.m5), s.m6);
    } else if (piece == 3) {
      s.mr = max_xor32(s.mr);
    } else if (piece == 4) {
      const float mt = s.mr * scale_log2;
      if (m_ref == -INFINITY) m_ref = mt;  // nothing accumulated yet for this head
      over = over || (mt > m_ref + kHead);
      s.neg = m_ref == -INFINITY ? 0.f : -m_ref;  // all masked so far: p = 0 anyway
      s.psum = 0.f;
    } else if (piece <= 20) {
      // one transcendental per piece: it takes a quarter-rate VALU slot
      const int r = piece - 5;
      // v_exp_f32: results below 2^-126 may flush to zero, negligible against l >= 1
      const float pr = __builtin_amdgcn_exp2f(fmaf(sc[r], scale_log2, s.neg));
      s.psum += pr;
      sc[r] = pr;
    } else if (piece <= 24) {
      const int r = 4 * (piece - 21);
#pragma unroll
      for (int e = 0; e < 4; ++e) s.pf[r >> 3][(r & 7) + e] = static_cast<__bf16>(sc[r + e]);
    } else {
      l_part += s.psum;
      sh.p[par][w][0][lane] = s.pf[0];
      sh.p[par][w][1][lane] = s.pf[1];
    }
  };
  auto mask_tail = [&](f32x16& sc, int nvalid) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (8 * (r >> 2) + 4 * hi + (r & 3) >= nvalid) sc[r] = -INFINITY;
  };
  auto softmax_all = [&](f32x16 sc, int nvalid, int par) __attribute__((always_inline)) {
    if (nvalid < kTileTok) mask_tail(sc, nvalid);
    SoftState s;
#pragma unroll
    for (int i = 0; i < kSoftPieces; ++i) soft_piece(i, sc, s, par);
  };

  // Rows of a partial tile past the history are zeroed in LDS before its P · V (their scores
  // are masked, but 0 x NaN would still poison O).
  auto zero_tail = [&](char* cur, int nvalid) __attribute__((always_inline)) {
    const int from = nvalid * kChunks, to = kTileChunks;
    for (int c = from + static_cast<int>(threadIdx.x); c < to; c += NW * 64)
      *reinterpret_cast<uint4*>(cur + 16 * c) = make_uint4(0u, 0u, 0u, 0u);
  };

  // ---- O[heads x wave's latent columns] += P · V for one tile, 16 positions per K-step,
  // with the softmax pieces of the next tile's scores `sc` between the products.
  auto pv = [&](const char* cur, int par, f32x16& sc, int npar) __attribute__((always_inline)) {
    SoftState s;
    bf16x8 pa[2][NW];
    i16x4 va[kVPre + 1][2];  // V fragments of kVPre + 1 (k2, db) steps: [buffer][rb]
    auto read_v = [&](int step, i16x4 (&dst)[2]) __attribute__((always_inline)) {
      const int n2 = step / kDB, ndb = step % kDB;
      const char* vp = cur + 16 * n2 * kRowBytes + (ndb >> 1) * 128;
      dst[0] = lds_read_tr(vp + vt[ndb & 1][0]);
      dst[1] = lds_read_tr(vp + vt[ndb & 1][1]);
    };
#pragma unroll
    for (int hb = 0; hb < NW; ++hb) pa[0][hb] = sh.p[par][hb][0][lane];
#pragma unroll
    for (int st = 0; st < kVPre; ++st) read_v(st, va[st]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kPV; ++i) {
      const int k2 = i / (kDB * NW), db = (i / NW) % kDB, hb = i % NW;
      const int step = i / NW;
      const int buf = step % (kVPre + 1);
      if (hb == 0 && step + kVPre < 2 * kDB) read_v(step + kVPre, va[(step + kVPre) % (kVPre + 1)]);
      if (i == kPV / 4) {
#pragma unroll
        for (int h2 = 0; h2 < NW; ++h2) pa[1][h2] = sh.p[par][h2][1][lane];
      }
      const bf16x8 vf = __builtin_bit_cast(
          bf16x8, __builtin_shufflevector(va[buf][0], va[buf][1], 0, 1, 2, 3, 4, 5, 6, 7));
      mfma_o(o[hb * kDB + db], pa[k2][hb], vf);
      // pieces start two products in, once the last score product has landed
      if (i >= 2 && i - 2 < kSoftPieces) soft_piece(i - 2, sc, s, npar);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = kPV - 2; i < kSoftPieces; ++i) soft_piece(i, sc, s, npar);
  };

  // ---- pipeline. Iteration t: tile t+1 has landed, tiles t+2 and t+3 are in flight (t+3
  // issued into the slot tile t-1 used), the scores of tile t+1 are formed, then P · V of
  // tile t runs with the softmax of tile t+1 spread between its products.
  // valid positions of the tiles after the current one: nv1 (t+1), nv2 (t+2)
  int nv1 = 0, nv2 = 0;
  {
    int nv0;
    issue_tile(tile_src(t0, &nv0), ring[0]);
    // vector memory completes in issue order: the query loads land before tiles 1 and 2, and
    // the compiler's waits for them (which do not count the copies) stay conservative
    {
      const char* qp = reinterpret_cast<const char*>(q_abs) +
                       (row0 + 32 * w + l32) * kRowBytes + hi * 16;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
    }
    if (ntiles > 1) issue_tile(tile_src(t0 + kTileTok, &nv1), ring[1]);
    if (ntiles > 2) issue_tile(tile_src(t0 + 2 * kTileTok, &nv2), ring[2]);
    if (ntiles > 2)
      wait_dma<2 * kDma>();
    else if (ntiles > 1)
      wait_dma<kDma>();
    else
      wait_dma<0>();
    __syncthreads();
    softmax_all(scores(ring[0], nullptr, 0u), nv0, 0);
    if (nv0 < kTileTok) zero_tail(ring[0], nv0);
  }

  // block and in-block offset of tile t+3, advanced by one tile per iteration
  int jb3 = (t0 + 3 * kTileTok) / bs;
  int off3 = t0 + 3 * kTileTok - jb3 * bs;
  for (int t = 0; t < ntiles; ++t) {
    const int slot = t & (kSlots - 1);
    const int nslot = (t + 1) & (kSlots - 1);
    const int pos0 = t0 + t * kTileTok;
    // tile t+1 has landed (tile t+2 may still be in flight); after the barrier P(t) and the
    // zeroed tail of tile t are visible to every wave and the slot of tile t-1 is free
    if (t + 2 < ntiles)
      wait_dma<kDma>();
    else
      wait_dma<0>();
    __syncthreads();
    int nv3 = 0;
    const char* src3 =
        t + 3 < ntiles ? tile_src_at(pos0 + 3 * kTileTok, jb3, off3, &nv3) : nullptr;
    off3 += kTileTok;
    if (off3 >= bs) {
      off3 -= bs;
      ++jb3;
    }
    // One body for every iteration (separate paths would split the query registers' live
    // ranges): on the last tile the next slot holds stale data, and with no valid position
    // the mask turns every score into -inf, which leaves m_ref, l and the flag unchanged.
    const int nv_next = t + 1 < ntiles ? nv1 : 0;
    nv1 = nv2;
    nv2 = nv3;
    f32x16 sc = scores(ring[nslot], src3, lds_addr(ring[(t + 3) & (kSlots - 1)]) + w * 64 * 16);
    if (nv_next < kTileTok) mask_tail(sc, nv_next);
    pv(ring[slot], t & 1, sc, (t + 1) & 1);
    // zeroed before the next barrier; other waves may still be reading these rows for their
    // scores, which are masked anyway
    if (t + 1 < ntiles && nv_next < kTileTok) zero_tail(ring[nslot], nv_next);
  }

  // ---- partials: o / l and m_ref + log2(l) per head, plus the recompute flag.
  // The last O products must have landed before VALU reads of O: 32 wait states, more than
  // any matrix-core result latency.
  asm volatile("s_nop 15\n\ts_nop 15"
               : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                 "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]),
                 "+a"(o[12]), "+a"(o[13]), "+a"(o[14]), "+a"(o[15]));
  const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
  const bool wover = __builtin_amdgcn_ballot_w64(over) != 0;
  Tail<NW>& tl = *reinterpret_cast<Tail<NW>*>(ring[0]);
  __syncthreads();  // every wave is done with the ring
  if (lane == 0) tl.over[w] = wover ? 1 : 0;
  if (lane < 32) {
    const int h = 32 * w + lane;
    tl.inv_l[h] = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    part_lse[prow0 + h] = l_tot > 0.f ? m_ref + log2f(l_tot) : -INFINITY;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int any = 0;
#pragma unroll
    for (int j = 0; j < NW; ++j) any |= tl.over[j];
    redo[split_id] = any;
  }
  // O / l leaves through the ring one 32-head block at a time (rows padded by 32 bytes so the
  // two half-waves' rows fall on different banks) and is written as bf16 with 16-byte stores.
  constexpr int kStageRow = kLat * 4 + 32;
  char* stage = ring[0] + 1024;  // after the Tail
  static_assert(1024 + 32 * kStageRow <= kSlots * kTileBytes, "stage fits in the ring");
  static_assert(sizeof(Tail<NW>) <= 1024, "tail fits before the stage");
  uint16_t* dst = part_o + prow0 * kLat;
#pragma unroll
  for (int hb = 0; hb < NW; ++hb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hl = 8 * (r >> 2) + 4 * hi + (r & 3);
      const float il = tl.inv_l[32 * hb + hl];
#pragma unroll
      for (int db = 0; db < kDB; ++db)
        *reinterpret_cast<float*>(stage + hl * kStageRow + ((kLat / NW) * w + 32 * db + l32) * 4) =
            o[hb * kDB + db][r] * il;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 32 * (kLat / 8); e += NW * 64) {
      const int row = e / (kLat / 8), c8 = e - row * (kLat / 8);
      const float4 lo = *reinterpret_cast<const float4*>(stage + row * kStageRow + 32 * c8);
      const float4 up = *reinterpret_cast<const float4*>(stage + row * kStageRow + 32 * c8 + 16);
      *reinterpret_cast<uint4*>(dst + (32 * hb + row) * kLat + 8 * c8) =
          make_uint4(pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w), pack_bf16x2(up.x, up.y),
                     pack_bf16x2(up.z, up.w));
    }
    __syncthreads();
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
                              void* part_o, float* part_lse, int* redo, SplitPlan* plan,
                              hipStream_t s) {
  const float scale_log2 = softmax_scale_of(d) * 1.4426950408889634f;
  const dim3 grid = plan != nullptr ? dim3(kPlanSlots) : dim3(n_split, s_q, batch);
#define MLA_LAUNCH(NW_)                                                                      \
  hipLaunchKernelGGL(decode_mfma_kernel<NW_>, grid, dim3(64 * NW_), 0, s,                     \
                     static_cast<const uint16_t*>(q_abs), static_cast<const uint16_t*>(cache), \
                     table, seq_lens, num_blocks, max_blocks, d.block_size, s_q, n_split,      \
                     scale_log2, static_cast<uint16_t*>(part_o), part_lse, redo, batch, plan)
  switch (d.n_heads) {
    case 128: MLA_LAUNCH(4); break;
    case 64: MLA_LAUNCH(2); break;
    default: MLA_LAUNCH(1); break;
  }
#undef MLA_LAUNCH
  return hipGetLastError();
}

}  // namespace mla
