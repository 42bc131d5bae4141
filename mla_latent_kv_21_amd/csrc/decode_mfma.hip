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
constexpr int kLatSteps = kLat / 16;              // 32 of them over the latent part
constexpr int kRopeSteps = kKSteps - kLatSteps;   // 4 over the rotary part
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
  bf16x8 qr[NW][kRopeSteps][64];  // rotary part of the queries (B operands of the last steps)
  float inv_l[NW * 32];
  int over[NW];            // a head of the wave outgrew its reference
};

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
  // K-step ks covers row elements [16 ks + 8 hi, +8). The latent steps stay in registers for
  // the whole split; the rotary steps are parked in LDS to leave registers for the pipeline.
  bf16x8 qf[kLatSteps];
  {
    const char* qp = reinterpret_cast<const char*>(a.q_abs) +
                     (row0 + 32 * w + l32) * kRowBytes + hi * 16;
#pragma unroll
    for (int ks = 0; ks < kLatSteps; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
#pragma unroll
    for (int r = 0; r < kRopeSteps; ++r)
      sh.qr[w][r][lane] = *reinterpret_cast<const bf16x8*>(qp + (kLatSteps + r) * 32);
  }

  // Per-lane LDS byte offsets inside a ring slot; the rest of every swizzled address is a
  // compile-time constant carried in the instruction's offset field.
  //  scores: position l32, chunk 8g + 2u + hi -> qb[u] + 128 g
  int qb[kGrp];
#pragma unroll
  for (int u = 0; u < kGrp; ++u) qb[u] = l32 * kRowBytes + (((2 * u + hi) ^ (l32 & 7)) << 4);
  //  values: position 16 k2 + 8 (e>>2) + 4 hi + (e&3), latent column (512/NW) w + 32 db + l32
  //  -> vb[db&1][e&3] + (16 k2 + 8 (e>>2)) * 1152 + (db>>1) * 128
  int vb[2][4];
#pragma unroll
  for (int dp = 0; dp < 2; ++dp)
#pragma unroll
    for (int e3 = 0; e3 < 4; ++e3)
      vb[dp][e3] = (4 * hi + e3) * kRowBytes + (((4 * dp + (l32 >> 3)) ^ (4 * hi + e3)) << 4) +
                   2 * (l32 & 7) + (8 / NW) * w * 128;

  f32x16 o[NW * kDB];
#pragma unroll
  for (int j = 0; j < NW * kDB; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[j][r] = 0.f;
  float m_ref = -INFINITY;  // reference max (log2 units) of head 32w + l32
  float l_part = 0.f;       // this lane's share of the softmax denominator
  bool over = false;
  const int ntiles = cdiv(t1 - t0, kTileTok);

  issue_tile<NW>(a, ring[0], b, t0, w, lane);
  if (ntiles > 1) issue_tile<NW>(a, ring[1], b, t0 + kTileTok, w, lane);
  wait_dma();
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int slot = t % 3;
    const char* cur = ring[slot];
    const int pos0 = t0 + t * kTileTok;
    const int nvalid = tile_valid(a, b, pos0, t1);
    // ---- scores S^T[position][head] over the 576-wide rows; fragments are read one group
    // ahead of their MFMAs (same-opcode accumulation into one register set is forwarded).
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
    {
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
          const bf16x8 qv = ks < kLatSteps ? qf[ks < kLatSteps ? ks : 0] : sh.qr[w][ks - kLatSteps][lane];
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cf[u], qv, sc, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kGrp; ++u) cf[u] = nf[u];
      }
    }
    // ---- softmax numerators against the head's fixed reference m_ref (log2 units): the
    // first finite tile max. A tile exceeding it by more than kHead marks the split for
    // recomputation by the portable kernel instead of rescaling O, so O is only ever
    // touched by MFMAs here.
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tp = 8 * (r >> 2) + 4 * hi + (r & 3);
      sc[r] = tp < nvalid ? sc[r] * a.scale_log2 : -INFINITY;
      mt = fmaxf(mt, sc[r]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    if (m_ref == -INFINITY) m_ref = mt;  // nothing accumulated yet for this head
    over = over || (mt > m_ref + kHead);
    float psum = 0.f;
    bf16x8 pf[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = sc[r] == -INFINITY ? 0.f : exp2f(sc[r] - m_ref);
      psum += p;
      pf[r >> 3][r & 7] = static_cast<__bf16>(p);
    }
    l_part += psum;
    const int par = t & 1;
    sh.p[par][w][0][lane] = pf[0];
    sh.p[par][w][1][lane] = pf[1];
    __builtin_amdgcn_sched_barrier(0);
    // The next tile's loads land here, and P becomes visible to every wave.
    wait_dma();
    __syncthreads();
    if (t + 2 < ntiles) issue_tile<NW>(a, ring[slot == 0 ? 2 : slot - 1], b, pos0 + 2 * kTileTok, w, lane);
    __builtin_amdgcn_sched_barrier(0);
    // ---- O[heads x wave's latent columns] += P · V, one K-step (16 positions) at a time
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      bf16x8 pa[NW];
#pragma unroll
      for (int hb = 0; hb < NW; ++hb) pa[hb] = sh.p[par][hb][k2][lane];
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        bf16x8 vf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tp = 16 * k2 + 8 * (e >> 2) + 4 * hi + (e & 3);
          const __bf16 x = *reinterpret_cast<const __bf16*>(
              cur + vb[db & 1][e & 3] + (16 * k2 + 8 * (e >> 2)) * kRowBytes + (db >> 1) * 128);
          vf[e] = tp < nvalid ? x : static_cast<__bf16>(0.f);
        }
#pragma unroll
        for (int hb = 0; hb < NW; ++hb)
          o[hb * kDB + db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[hb], vf, o[hb * kDB + db],
                                                                     0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
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
