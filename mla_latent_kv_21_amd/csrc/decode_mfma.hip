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
//  * one workgroup per (split, query, sequence) of NW = 4 waves and H/32 blocks of 32 heads
//    (fewer waves than SIMDs would leave matrix cores idle while one wave works through a
//    tile): wave w forms the scores of block w % (H/32), at H = 64 two waves alike; at H = 32
//    the four waves split the block's score contraction and add their partial sums through
//    LDS. Wave w owns latent columns [128w, 128w+128) of all heads for the output;
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
//    and is exchanged through LDS (at H = 32 every wave holds the whole P itself);
//    O[H x 512/NW] += P · V with V read by transposing LDS reads from the same tile;
//  * the loop body is scheduled by hand: the scores of tile t+1 run with their LDS reads
//    several steps ahead, then P · V of tile t runs with the softmax of tile t+1 spread
//    between its products, so the matrix cores are fed while the VALU and LDS work;
//  * each split writes (O / l as bf16, m + log2 l) partials; the merge kernel combines them.
//
// e4m3 variant (H = 128): rows of d_c + d_r bytes with one fp32 power-of-two scale per slot.
// Tiles (18,432 B + 128 B of scales) stream into a 3-slot staging ring, swizzled like the bf16
// ring; at the top of each iteration the staged tile is dequantised once (byte x scale, exact
// in bf16) into one of two bf16 slots and published by a second barrier, after which the
// scores and P · V are the bf16 kernel's own, so the results equal the bf16 kernel's on the
// dequantised rows bit for bit.
#include "common.hpp"
#include "launch.hpp"
#include "mfma_util.hpp"
#include "plan.hpp"

namespace mla {
namespace {

using namespace mfma;

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
// e4m3 rows (d_c + d_r bytes, one fp32 scale per position): 32-position tiles of 18,432 bytes
// plus their 128 bytes of scales stream into a 3-slot staging ring placed after two bf16
// value slots (which hold only the dequantised latent columns the P · V product reads)
constexpr int kF8RowBytes = kRowElems;                      // 576
constexpr int kF8Chunks = kF8RowBytes / 16;                 // 36
constexpr int kF8TileBytes = kTileTok * kF8RowBytes;        // 18,432
constexpr int kF8SlotBytes = kF8TileBytes + 4 * kTileTok;   // + the tile's 32 scales
constexpr int kF8Slots = 3;
constexpr int kF8Base = 2 * kTileBytes;                     // staging after two bf16 slots
constexpr int kDma8 = 5;                                    // copies per wave per fp8 tile
constexpr int kPreF8 = 6;                                   // score fragments ahead (e4m3)
static_assert(kF8Base + kF8Slots * kF8SlotBytes <= kSlots * kTileBytes, "fp8 staging fits");

// Physical 16-byte chunk of logical chunk c in row t of an e4m3 staging tile: XOR-swizzled
// inside groups of four by bits 2..3 of the row, so that the score reads (8 bytes per lane,
// one chunk of all 32 rows) spread evenly over the banks.
__host__ __device__ constexpr int swz8(int t, int c) { return (c & ~3) | ((c & 3) ^ ((t >> 2) & 3)); }

// A device address as a wave-uniform value (so that asm operands can take it in SGPRs).
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(v));
  const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(v >> 32));
  return reinterpret_cast<const char*>((static_cast<unsigned long long>(hi) << 32) | lo);
}

// Physical 16-byte chunk of logical chunk c in tile row t is c ^ swz(t). swz is a linear map
// of the row's low four bits into three bits (a row's 72 chunks stay in their groups of 8).
// It is chosen so that the score reads (16 bytes per lane, 32 rows x one chunk pair) and the
// transposing value reads (8 bytes per lane, 4 rows x 2 chunks per 16 lanes) hit distinct
// banks within every 128- and 256-byte LDS beat.
__host__ __device__ constexpr int swz(int t) {
  return ((t & 1) ? 3 : 0) ^ ((t & 2) ? 4 : 0) ^ ((t & 4) ? 2 : 0) ^ ((t & 8) ? 1 : 0);
}

// O += A · B with O held in accumulation registers (AGPRs). The score products use the
// compiler's MFMA in its VGPR form (this file is built with MFMA results in VGPRs), so that
// O (256 AGPRs) and the score accumulator never compete for one register file. The compiler
// does not track this instruction's hazards: the leading s_nop covers a VALU write of A or B
// just before it (two wait states); O is only ever written by this instruction, and is read
// only after the explicit wait that follows the main loop.
__device__ __forceinline__ void mfma_o(f32x16& o, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(b));
}

// Waves of a workgroup with HB blocks of 32 heads: always four (with fewer than four blocks,
// wave w takes block w % HB for the scores, each block's scores formed by 4 / HB waves).
__host__ __device__ constexpr int waves_of(int) { return 4; }

template <int HB>
struct Shared {
  bf16x8 p[2][HB][2][64];         // P fragments: [parity][head block][K-step][lane]
};
// H = 32: the four waves' partial scores of one tile, [wave][register quad][lane]
template <>
struct Shared<1> {
  float4 s[4][4][64];
};
// After the loop the ring is free and holds the per-head 1/l and the waves' flags.
template <int HB>
struct Tail {
  float inv_l[HB * 32];
  int over[waves_of(HB)];         // a head of the wave outgrew its reference
};

struct SoftState {
  float m1, m2, m3, m4, m5, m6, mr, neg, psum;
  bf16x8 pf[2];
};

// kFp8: the cache rows are e4m3 bytes with one fp32 power-of-two scale per position
// (`scales`, indexed like the cache slots); see the e4m3 variant above.
// kNT: the cache-tile copies carry the non-temporal hint (H = 128 with one query row per
// sequence, where each tile has one reader).
// kApp: a decode step whose s_q new tokens (positions L - s_q .. L - 1 of each sequence, token
// n = b s_q + i) were projected but not yet written: every workgroup first forms the new rows
// inside its own range from the projection's partial sums (`app`), exactly as the append's
// finalize does (with kFp8, quantised to e4m3 bytes and a scale by the finalize's rule),
// stores them at their slots and waits for the stores before its copies read them.
// Workgroups of several query rows may form the same row; they store the same bytes.
template <int HB, bool kFp8, bool kApp, bool kNT>
__global__ __launch_bounds__(waves_of(HB) * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mfma_kernel(const uint16_t* __restrict__ q_abs, const uint16_t* __restrict__ cache,
                        const float* __restrict__ scales, StepRows app,
                        const int32_t* __restrict__ table, const int32_t* __restrict__ lens,
                        int num_blocks, int max_blocks, int bs, int s_q, int n_split,
                        float scale_log2, uint16_t* __restrict__ part_o,
                        float* __restrict__ part_lse, int* __restrict__ redo, int batch,
                        SplitPlan* __restrict__ plan_out) {
  constexpr int NW = waves_of(HB);                  // waves
  constexpr bool kDup = NW > HB;                    // several waves form each block's scores
  constexpr bool kRegP = HB == 1;                   // P stays in registers (one head block)
  // H = 32: the score contraction is split over the four waves (a quarter of the 576-wide
  // rows each, 9 K-steps), the partial scores added through LDS in wave order
  constexpr bool kKS = HB == 1;
  constexpr int kQS = kKS ? kKSteps / NW : kKSteps;  // K-steps of the wave's score products
  constexpr int H = HB * 32;
  constexpr int kDB = 16 / NW;                      // 32-column latent blocks per wave
  constexpr int kPV = 2 * kDB * HB;                 // P · V products per tile per wave
  constexpr int kDma = kTileChunks / (NW * 64);     // copies per wave per tile
  static_assert(kDma <= kKSteps, "copies are spread over the score K-steps");
  __shared__ __attribute__((aligned(16))) char ring[kSlots][kTileBytes];
  __shared__ Shared<HB> sh;
  static_assert(sizeof(ring) + sizeof(Shared<HB>) <= 160 * 1024, "LDS");
  // bf16 tile slots in use: four (two in flight, two computed on) or, with e4m3 rows, two
  // (the staging ring holds the tiles in flight)
  constexpr int kBMask = (kFp8 ? 2 : kSlots) - 1;
  auto stage8 = [&](int i) -> char* {
    return reinterpret_cast<char*>(ring) + kF8Base + (i % kF8Slots) * kF8SlotBytes;
  };
  static_assert(!kFp8 || HB == 4, "the e4m3 copy plan is laid out for four waves, H = 128");

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
    // Workgroup x runs on XCD x % 8 (workgroups are dealt to the XCDs in turn), so XCD c takes
    // the contiguous slots [32 c, 32 c + 32): the s_q query rows of one sequence, whose slots
    // are adjacent, then stream the same cache tiles through one L2, which serves all but the
    // first read of each tile.
    static_assert(kPlanSlots % 8 == 0, "one slot range per XCD");
    const int slot = (blockIdx.x & 7) * (kPlanSlots / 8) + (blockIdx.x >> 3);
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

  if constexpr (kApp) {
    static_assert(HB == 4, "new rows are formed by four waves, H = 128");
    const int L = __builtin_amdgcn_readfirstlane(lens[b]);
    const int n_tok = batch * s_q;
    float* ys = reinterpret_cast<float*>(ring[3]);  // the ring is not in use yet
    float* red = ys + kRowElems;
    const float* __restrict__ yp = app.y_part;
    const uint16_t* __restrict__ gam = static_cast<const uint16_t*>(app.gamma);
    uint16_t* __restrict__ cw = static_cast<uint16_t*>(app.cache);
    const int first_new = max(t0, L - s_q);
    for (int p = first_new; p < t1; ++p) {
      const int n = b * s_q + (p - (L - s_q));
      const int64_t slot = cache_slot(table, max_blocks, bs, num_blocks, b, p);
      // column c = threadIdx.x + 256 j: the partial sums in the fixed order k = 0, 1, ...
      // The three columns' partials are requested together, kYB per column at a time (one
      // round trip for d_model <= 8,192): only this workgroup forms the row, and its copies
      // wait for it.
      constexpr int kYB = 32;
      float y[3];
#pragma unroll
      for (int j = 0; j < 3; ++j) y[j] = 0.f;
      for (int kk = 0; kk < app.n_ksplit; kk += kYB) {
        float v[3][kYB];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const int c = threadIdx.x + 256 * j;
#pragma unroll
          for (int u = 0; u < kYB; ++u)
            v[j][u] = c < kRowElems && kk + u < app.n_ksplit
                          ? yp[(static_cast<int64_t>(kk + u) * n_tok + n) * kRowElems + c]
                          : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
          for (int u = 0; u < kYB; ++u)
            if (kk + u < app.n_ksplit) y[j] += v[j][u];
      }
      // the latent's sum of squares: 64-column block w + 4 j by a butterfly over wave w, then
      // the eight blocks in order
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float s2 = wave_sum(square_rn(y[j]));
        if (lane == 0) red[w + 4 * j] = s2;
      }
      __syncthreads();
      float ss = 0.f;
#pragma unroll
      for (int blk = 0; blk < kLat / 64; ++blk) ss += red[blk];
      const float inv = 1.0f / sqrtf(ss / static_cast<float>(kLat) + app.eps);
      // the rotary pair of column 512 + threadIdx.x (wave 0) is held by lanes 2 jj, 2 jj + 1
      const float partner = __shfl_xor(y[2], 1, 64);
      if constexpr (kFp8) {
        // the values the bf16 row would hold, then their e4m3 bytes and the row's scale
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int c = threadIdx.x + 256 * j;
          const float v = bf16_to_f32(f32_to_bf16(y[j] * inv * bf16_to_f32(gam[c])));
          ys[c] = v;
          amax = fmaxf(amax, fabsf(v));
        }
        if (threadIdx.x < kRowElems - kLat) {
          const int jj = threadIdx.x >> 1;
          float cs, sn, u, v;
          rope_cos_sin(p, jj, kRowElems - kLat, app.base, &cs, &sn);
          const bool even = (threadIdx.x & 1) == 0;
          rope_rotate(even ? y[2] : partner, even ? partner : y[2], cs, sn, &u, &v);
          const float r = bf16_to_f32(f32_to_bf16(even ? u : v));
          ys[kLat + threadIdx.x] = r;
          amax = fmaxf(amax, fabsf(r));
        }
        amax = wave_max(amax);
        if (lane == 0) red[8 + w] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(red[8], red[9]), fmaxf(red[10], red[11]));
        const int e = e4m3_scale_exp(amax);
        const float rs = ldexpf(1.f, -e);
        if (slot >= 0) {
          if (threadIdx.x < kRowElems / 4) {
            const float* v4 = ys + 4 * threadIdx.x;
            reinterpret_cast<unsigned*>(static_cast<uint8_t*>(app.cache) + slot * kRowElems)
                [threadIdx.x] = e4m3_pack4(v4[0] * rs, v4[1] * rs, v4[2] * rs, v4[3] * rs);
          }
          if (threadIdx.x == 0) app.scale[slot] = ldexpf(1.f, e);
        }
      } else if (slot >= 0) {
        uint16_t* row = cw + slot * kRowElems;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int c = threadIdx.x + 256 * j;
          row[c] = f32_to_bf16(y[j] * inv * bf16_to_f32(gam[c]));
        }
        if (threadIdx.x < kRowElems - kLat) {
          const int jj = threadIdx.x >> 1;
          float cs, sn, u, v;
          rope_cos_sin(p, jj, kRowElems - kLat, app.base, &cs, &sn);
          const bool even = (threadIdx.x & 1) == 0;
          rope_rotate(even ? y[2] : partner, even ? partner : y[2], cs, sn, &u, &v);
          row[kLat + threadIdx.x] = f32_to_bf16(even ? u : v);
        }
      }
      __syncthreads();  // red is free for the next row
    }
    if (first_new < t1) {
      // every wave's stores are done before any wave's copies read the rows
      wait_vm<0>();
      __syncthreads();
    }
  }

  const int l32 = lane & 31, hi = lane >> 5;
  const int hbw = w % HB;  // the wave's head block for the scores

  // Absorbed queries of this wave's 32 heads as MFMA B operands, in registers for the whole
  // split: lane -> head 32w + l32, K-step ks covers row elements [16 ks + 8 hi, +8). Loaded
  // after the first tile's copies are issued.
  bf16x8 qf[kQS];
  const int ks0 = kKS ? kQS * w : 0;  // the wave's first score K-step

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

  constexpr int kNO = HB * kDB;  // O accumulators per wave (16; 8 at H = 64, 4 at H = 32)
  f32x16 o[kNO];
#pragma unroll
  for (int j = 0; j < kNO; ++j)
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
  constexpr int kRB = kFp8 ? kF8RowBytes : kRowBytes;  // bytes per cache row in memory
  const int64_t blk_bytes = static_cast<int64_t>(bs) * kRB;
  int64_t tile_first_slot = 0;  // cache slot of the last tile looked up (e4m3: its scales)
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
    if constexpr (kFp8) tile_first_slot = static_cast<int64_t>(ok ? id : 0) * bs + off;
    return reinterpret_cast<const char*>(cache) + (ok ? id : 0) * blk_bytes + off * kRB;
  };
  auto tile_src = [&](int pos0, int* nvalid) -> const char* {
    const int jb = pos0 / bs;
    return tile_src_at(pos0, jb, pos0 - jb * bs, nvalid);
  };
  // At H = 128 with one query row per sequence every cache tile is copied once, by one
  // workgroup, and the copies carry the non-temporal hint (measured faster there: the
  // long-128k step by ≈ 3 %). With several query rows per sequence (s_q > 1) the rows'
  // workgroups of one split read the same tiles on one XCD and the copies keep the default
  // policy, so that a tile stays in L2 for the other rows; with fewer head blocks the
  // default policy measured as fast or faster.
  auto issue_tile = [&](const char* src, char* slot) __attribute__((always_inline)) {
    const unsigned lbase = lds_addr(slot) + w * 64 * 16;
#pragma unroll
    for (int j = 0; j < kDma; ++j) dma16<kNT>(src, doff[j], lbase + j * NW * 64 * 16);
  };
  // Copy j of a tile issued from inside the score loop: the copies of the four waves then
  // spread over the score phase instead of queueing at the vector-memory unit together.
  auto issue_part = [&](const char* src, unsigned lbase, int j) __attribute__((always_inline)) {
    if (src != nullptr) dma16<kNT>(src, doff[j], lbase + j * NW * 64 * 16);
  };
  // e4m3 tiles: LDS chunk p of a staging slot (row p / 36, physical chunk p % 36) is filled
  // from the row's logical chunk swz8(row, p % 36) (the swizzle is its own inverse). Copy
  // j < 4 fills chunks (4 j + w) 64 + lane; copy 4 fills chunks 1024 .. 1151 (waves 0 and 1)
  // or the tile's 32 scales (lanes 0..7 of waves 2 and 3, the same bytes twice), so that every
  // wave issues the same number of copies per tile.
  unsigned doff8[kFp8 ? kDma8 : 1];
  if constexpr (kFp8) {
#pragma unroll
    for (int j = 0; j < kDma8; ++j) {
      const int p = j < 4 ? (4 * j + w) * 64 + lane : 1024 + w * 64 + lane;
      const int t = p / kF8Chunks, pc = p - t * kF8Chunks;
      doff8[j] = j < 4 || w < 2 ? static_cast<unsigned>(t * kF8RowBytes + 16 * swz8(t, pc))
                                : static_cast<unsigned>(lane * 16);
    }
  }
  auto issue_part8 = [&](const char* src, const char* ssrc, unsigned lbase, int j)
                         __attribute__((always_inline)) {
    if (src == nullptr) return;
    if (j < 4) {
      dma16<kNT>(src, doff8[j], lbase + (4 * j + w) * 64 * 16);
    } else if (w < 2) {
      dma16<kNT>(src, doff8[j], lbase + (1024 + w * 64) * 16);
    } else if (lane < 8) {
      dma16<kNT>(ssrc, doff8[j], lbase + kF8TileBytes);
    }
  };
  // the tile's scales in memory (e4m3 rows), from the slot tile_src_at just looked up
  auto scales_src = [&]() -> const char* {
    return uniform_ptr(reinterpret_cast<const char*>(scales + tile_first_slot));
  };
  // e4m3 -> bf16 of four bytes times a power-of-two scale (exact), element 0 in the low half
  auto cvt4 = [&](unsigned x, float sc, unsigned* lo, unsigned* hi) __attribute__((always_inline)) {
    *lo = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, sc, false));
    *hi = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, sc, true));
  };
  // A staged e4m3 tile dequantised into a bf16 tile slot, in the swizzled layout the scores
  // and P · V read: thread 8 t + s converts logical chunks s, s + 8, ... of row t (16 values
  // each, byte x scale, exact in bf16) into bf16 chunks 2 c and 2 c + 1; rows past nvalid
  // become zeros.
  auto dequant = [&](const char* f8, char* bt, int nvalid) __attribute__((always_inline)) {
    const int t = threadIdx.x >> 3, s8 = threadIdx.x & 7;
    const float sc = *reinterpret_cast<const float*>(f8 + kF8TileBytes + 4 * t);
    const bool ok = t < nvalid;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const int c = s8 + 8 * k;
      if (k < 4 || c < kF8Chunks) {
        uint4 lo = make_uint4(0u, 0u, 0u, 0u), up = lo;
        if (ok) {
          const uint4 v = *reinterpret_cast<const uint4*>(f8 + t * kF8RowBytes + 16 * swz8(t, c));
          cvt4(v.x, sc, &lo.x, &lo.y);
          cvt4(v.y, sc, &lo.z, &lo.w);
          cvt4(v.z, sc, &up.x, &up.y);
          cvt4(v.w, sc, &up.z, &up.w);
        }
        *reinterpret_cast<uint4*>(bt + t * kRowBytes + (((2 * c) ^ swz(t)) << 4)) = lo;
        *reinterpret_cast<uint4*>(bt + t * kRowBytes + (((2 * c + 1) ^ swz(t)) << 4)) = up;
      }
    }
  };

  // ---- scores S^T[position][head] of one tile over the 576-wide rows, each fragment read
  // kPre products ahead of its MFMA.
  constexpr int kCopies = kFp8 ? kDma8 : kDma;
  // H = 32: byte offsets of the wave's K-steps in a tile (logical chunk 2 ks + hi of row l32)
  int koff[kKS ? kQS : 1];
  if constexpr (kKS) {
#pragma unroll
    for (int j = 0; j < kQS; ++j)
      koff[j] = l32 * kRowBytes + (((2 * (ks0 + j) + hi) ^ swz(l32)) << 4);
  }
  auto scores = [&](const char* cur, const char* dsrc, unsigned dlds, const char* ssrc)
                    __attribute__((always_inline)) -> f32x16 {
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
    if constexpr (kKS) {
      static_assert(kKSteps % NW == 0 && kDma == kQS, "one copy per K-step of the wave");
      bf16x8 af[kQS];
#pragma unroll
      for (int j = 0; j < kQS; ++j) af[j] = lds16(cur + koff[j]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < kQS; ++j) {
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[j], qf[j], sc, 0, 0, 0);
        issue_part(dsrc, dlds, j);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the partial sums through LDS; every wave adds the four in wave order (the same bits
      // in every wave). The previous tile's partials were read before the loop's barrier.
#pragma unroll
      for (int k = 0; k < 4; ++k)
        sh.s[w][k][lane] = make_float4(sc[4 * k], sc[4 * k + 1], sc[4 * k + 2], sc[4 * k + 3]);
      __syncthreads();
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 a = sh.s[0][k][lane], b = sh.s[1][k][lane], c = sh.s[2][k][lane],
                     d = sh.s[3][k][lane];
        sc[4 * k] = ((a.x + b.x) + c.x) + d.x;
        sc[4 * k + 1] = ((a.y + b.y) + c.y) + d.y;
        sc[4 * k + 2] = ((a.z + b.z) + c.z) + d.z;
        sc[4 * k + 3] = ((a.w + b.w) + c.w) + d.w;
      }
      return sc;
    } else {
      // fewer fragments ahead where the copy offsets take more registers (e4m3 rows)
      constexpr int kP = kFp8 ? kPreF8 : kPre;
      bf16x8 af[kP];
#pragma unroll
      for (int i = 0; i < kP; ++i) af[i] = lds16(cur + qb[i & 3] + 128 * (i >> 2));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const bf16x8 acur = af[ks % kP];
        const int nx = ks + kP;
        if (nx < kKSteps) af[ks % kP] = lds16(cur + qb[nx & 3] + 128 * (nx >> 2));
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(acur, qf[ks], sc, 0, 0, 0);
        // copies spread evenly over the K-steps (kCopies <= kKSteps)
        if ((ks * kCopies) / kKSteps != ((ks + 1) * kCopies) / kKSteps) {
          if constexpr (kFp8)
            issue_part8(dsrc, ssrc, dlds, (ks * kCopies) / kKSteps);
          else
            issue_part(dsrc, dlds, (ks * kCopies) / kKSteps);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      return sc;
    }
  };
  // ---- softmax numerators of one tile against the head's fixed reference m_ref (log2
  // units): the first finite tile max. A tile exceeding it by more than kHead marks the split
  // for exact recomputation instead of rescaling O, so O is only ever touched by MFMAs. The
  // numerators are left in P's LDS slot `par` as the A operand of the next P · V.
  // Split in pieces (compile-time numbers) so the unmasked case can be spread between the
  // P · V products.
  constexpr int kSoftPieces = 26;
  // with H = 32 the wave keeps P in registers: P of the tile P · V is working on (p_cur) and
  // of the next tile, formed by the softmax pieces meanwhile (p_next)
  bf16x8 p_cur[2], p_next[2];
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
      if constexpr (kRegP) {
        p_next[0] = s.pf[0];
        p_next[1] = s.pf[1];
      } else if (!kDup || w < HB) {  // one of the waves that formed the block's P
        sh.p[par][hbw][0][lane] = s.pf[0];
        sh.p[par][hbw][1][lane] = s.pf[1];
      }
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
    bf16x8 pa[2][HB];
    i16x4 va[kVPre + 1][2];  // V fragments of kVPre + 1 (k2, db) steps: [buffer][rb]
    auto read_v = [&](int step, i16x4 (&dst)[2]) __attribute__((always_inline)) {
      const int n2 = step / kDB, ndb = step % kDB;
      const char* vp = cur + 16 * n2 * kRowBytes + (ndb >> 1) * 128;
      dst[0] = lds_read_tr(vp + vt[ndb & 1][0]);
      dst[1] = lds_read_tr(vp + vt[ndb & 1][1]);
    };
    if constexpr (kRegP) {
      pa[0][0] = p_cur[0];
      pa[1][0] = p_cur[1];
    } else {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) pa[0][hb] = sh.p[par][hb][0][lane];
    }
#pragma unroll
    for (int st = 0; st < kVPre; ++st) read_v(st, va[st]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kPV; ++i) {
      const int k2 = i / (kDB * HB), db = (i / HB) % kDB, hb = i % HB;
      const int step = i / HB;
      const int buf = step % (kVPre + 1);
      if (hb == 0 && step + kVPre < 2 * kDB) read_v(step + kVPre, va[(step + kVPre) % (kVPre + 1)]);
      if constexpr (!kRegP) {
        if (i == kPV / 4) {
#pragma unroll
          for (int h2 = 0; h2 < HB; ++h2) pa[1][h2] = sh.p[par][h2][1][lane];
        }
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
    if constexpr (kFp8) {
      const char* src = tile_src(t0, &nv0);
      const unsigned lb = lds_addr(stage8(0));
      for (int j = 0; j < kDma8; ++j) issue_part8(src, scales_src(), lb, j);
    } else {
      issue_tile(tile_src(t0, &nv0), ring[0]);
    }
    // vector memory completes in issue order: the query loads land before tiles 1 and 2, and
    // the compiler's waits for them (which do not count the copies) stay conservative
    {
      const char* qp = reinterpret_cast<const char*>(q_abs) +
                       (row0 + 32 * hbw + l32) * kRowBytes + hi * 16;
#pragma unroll
      for (int ks = 0; ks < kQS; ++ks)
        qf[ks] = *reinterpret_cast<const bf16x8*>(qp + (ks0 + ks) * 32);
    }
    if constexpr (kFp8) {
      for (int i = 1; i < 3; ++i) {
        if (ntiles > i) {
          const char* src = tile_src(t0 + i * kTileTok, i == 1 ? &nv1 : &nv2);
          const unsigned lb = lds_addr(stage8(i));
          for (int j = 0; j < kDma8; ++j) issue_part8(src, scales_src(), lb, j);
        }
      }
    } else {
      if (ntiles > 1) issue_tile(tile_src(t0 + kTileTok, &nv1), ring[1]);
      if (ntiles > 2) issue_tile(tile_src(t0 + 2 * kTileTok, &nv2), ring[2]);
    }
    if (ntiles > 2)
      wait_vm<2 * kCopies>();
    else if (ntiles > 1)
      wait_vm<kCopies>();
    else
      wait_vm<0>();
    __syncthreads();
    if constexpr (kFp8) {
      dequant(stage8(0), ring[0], nv0);
      __syncthreads();
    }
    softmax_all(scores(ring[0], nullptr, 0u, nullptr), nv0, 0);
    if constexpr (kRegP) {
      p_cur[0] = p_next[0];
      p_cur[1] = p_next[1];
    }
    if constexpr (!kFp8) {
      if (nv0 < kTileTok) zero_tail(ring[0], nv0);
    }
  }

  // block and in-block offset of tile t+3, advanced by one tile per iteration
  int jb3 = (t0 + 3 * kTileTok) / bs;
  int off3 = t0 + 3 * kTileTok - jb3 * bs;
  for (int t = 0; t < ntiles; ++t) {
    const int slot = t & kBMask;
    const int nslot = (t + 1) & kBMask;
    const int pos0 = t0 + t * kTileTok;
    // tile t+1 has landed (tile t+2 may still be in flight); after the barrier P(t) and the
    // zeroed tail of tile t are visible to every wave and the slot of tile t-1 is free
    if (t + 2 < ntiles)
      wait_vm<kCopies>();
    else
      wait_vm<0>();
    __syncthreads();
    int nv3 = 0;
    const char* src3 =
        t + 3 < ntiles ? tile_src_at(pos0 + 3 * kTileTok, jb3, off3, &nv3) : nullptr;
    const char* ssrc3 = nullptr;
    if constexpr (kFp8) ssrc3 = src3 != nullptr ? scales_src() : nullptr;
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
    if constexpr (kFp8) {
      // staged tile t+1 dequantised into the bf16 slot tile t-1 used (every wave is past its
      // P · V), published by a second barrier; the copies of tile t+3 then go to the staging
      // slot of tile t, dequantised in the previous iteration
      if (t + 1 < ntiles) dequant(stage8(t + 1), ring[nslot], nv_next);
      __syncthreads();
    }
    const unsigned dlds = kFp8 ? lds_addr(stage8(t + 3))
                               : lds_addr(ring[(t + 3) & (kSlots - 1)]) + w * 64 * 16;
    f32x16 sc = scores(ring[nslot], src3, dlds, ssrc3);
    if (nv_next < kTileTok) mask_tail(sc, nv_next);
    pv(ring[slot], t & 1, sc, (t + 1) & 1);
    if constexpr (kRegP) {
      p_cur[0] = p_next[0];
      p_cur[1] = p_next[1];
    }
    // zeroed before the next barrier; other waves may still be reading these rows for their
    // scores, which are masked anyway
    if constexpr (!kFp8) {
      if (t + 1 < ntiles && nv_next < kTileTok) zero_tail(ring[nslot], nv_next);
    }
  }

  // ---- partials: o / l and m_ref + log2(l) per head, plus the recompute flag.
  // The last O products must have landed before VALU reads of O: 32 wait states, more than
  // any matrix-core result latency.
  if constexpr (kNO == 16)
    asm volatile("s_nop 15\n\ts_nop 15"
                 : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                   "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]),
                   "+a"(o[12]), "+a"(o[13]), "+a"(o[14]), "+a"(o[15]));
  else if constexpr (kNO == 8)
    asm volatile("s_nop 15\n\ts_nop 15"
                 : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                   "+a"(o[6]), "+a"(o[7]));
  else
    asm volatile("s_nop 15\n\ts_nop 15" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]));
  static_assert(kNO == 16 || kNO == 8 || kNO == 4, "the wait above names every accumulator");
  const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
  const bool wover = __builtin_amdgcn_ballot_w64(over) != 0;
  Tail<HB>& tl = *reinterpret_cast<Tail<HB>*>(ring[0]);
  __syncthreads();  // every wave is done with the ring
  if (lane == 0) tl.over[w] = wover ? 1 : 0;
  if (lane < 32 && w < HB) {  // (waves w and w + HB hold the same l)
    const int h = 32 * hbw + lane;
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
  static_assert(sizeof(Tail<HB>) <= 1024, "tail fits before the stage");
  uint16_t* dst = part_o + prow0 * kLat;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
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

bool mfma_step_fits(const mla_dims& d) {
  return d.dtype == MLA_BF16 && d.d_c == 512 && d.d_r == 64 && d.block_size % 32 == 0 &&
         d.n_heads == 128 && !(d.flags & MLA_FLAG_GENERIC_KERNELS);
}

bool mfma_decode_fp8_fits(const mla_dims& d) {
  return d.dtype == MLA_BF16 && d.d_c == 512 && d.d_r == 64 && d.block_size % 32 == 0 &&
         d.n_heads == 128;
}

bool mfma_decode_fits(const mla_dims& d) {
  return d.dtype == MLA_BF16 && d.d_c == 512 && d.d_r == 64 && d.block_size % 32 == 0 &&
         (d.n_heads == 32 || d.n_heads == 64 || d.n_heads == 128);
}

hipError_t launch_decode_mfma(const mla_dims& d, int batch, int s_q, const void* q_abs,
                              const void* cache, const float* scales, int num_blocks,
                              const int32_t* table, int max_blocks, const int32_t* seq_lens,
                              int n_split, void* part_o, float* part_lse, int* redo,
                              SplitPlan* plan, const StepRows* app, hipStream_t s) {
  const StepRows none{};
  const float scale_log2 = softmax_scale_of(d) * 1.4426950408889634f;
  const dim3 grid = plan != nullptr ? dim3(kPlanSlots) : dim3(n_split, s_q, batch);
#define MLA_LAUNCH1(HB_, FP8_, APP_, NT_)                                                    \
  hipLaunchKernelGGL((decode_mfma_kernel<HB_, FP8_, APP_, NT_>), grid, dim3(64 * waves_of(HB_)), \
                     0, s,                                                                       \
                     static_cast<const uint16_t*>(q_abs), static_cast<const uint16_t*>(cache), \
                     scales, app != nullptr ? *app : none, table, seq_lens, num_blocks,        \
                     max_blocks, d.block_size, s_q, n_split, scale_log2,                       \
                     static_cast<uint16_t*>(part_o), part_lse, redo, batch, plan)
  // H = 128: streaming copies when each tile has one reader (s_q = 1)
  const bool nt = s_q == 1;
#define MLA_LAUNCH(HB_, FP8_, APP_)    \
  do {                                 \
    if (nt)                            \
      MLA_LAUNCH1(HB_, FP8_, APP_, true);  \
    else                               \
      MLA_LAUNCH1(HB_, FP8_, APP_, false); \
  } while (0)
  if (app != nullptr && scales != nullptr) {
    MLA_LAUNCH(4, true, true);   // e4m3 rows formed in the core: H = 128
  } else if (app != nullptr) {
    MLA_LAUNCH(4, false, true);  // new rows formed in the core: H = 128 (mfma_step_fits)
  } else if (scales != nullptr) {
    MLA_LAUNCH(4, true, false);  // e4m3 rows: H = 128 only (mfma_decode_fp8_fits)
  } else {
    switch (d.n_heads) {
      case 128: MLA_LAUNCH(4, false, false); break;
      case 64: MLA_LAUNCH1(2, false, false, false); break;
      default: MLA_LAUNCH1(1, false, false, false); break;
    }
  }
#undef MLA_LAUNCH
#undef MLA_LAUNCH1
  return hipGetLastError();
}

}  // namespace mla
