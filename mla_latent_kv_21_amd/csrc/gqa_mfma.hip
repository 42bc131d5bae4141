// Split-K grouped-query decode over the expanded GQA cache on gfx950 matrix cores: bf16,
// D = D_v = 128, d_r = 64, any number of query rows (heads of one group x query tokens) in
// workgroups of 32: decode steps and, with the expanded cache of every head, prefill.
//
// What is computed is the GQA path of the GQLA summary (section 2, "Chemin GQA"): head h of
// group g scores [q_nope_h ; rotation(q_pe_h)] against the cached [K_g ; k_r] rows, takes the
// softmax (mkdocs.reaper.mx "Le mécanisme d'attention") and averages V_g. Decode is bound by
// reading the cache, so every cached byte a group needs is read from HBM once per step:
//
//  * one single-wave workgroup per (sequence, split, group); the G workgroups of one
//    (sequence, split) are numbered so that they run on one XCD, where they share k_r in L2;
//  * 32-position tiles of the group's K_g (256 B), V_g (256 B) and k_r (128 B) per position
//    (20 KiB, always inside one cache block) stream HBM -> LDS with global_load_lds_dwordx4
//    into a 2-slot ring: the next tile is in flight while one is used, and four workgroups
//    share a CU (more waves issuing copies beat a deeper ring per wave); the 16-byte chunks
//    of a row are XOR-swizzled by position so that the score reads and the transposing value
//    reads are bank-conflict free;
//  * S^T [32 positions x 32 rows] = [K_g | k_r] · Q^T with v_mfma_f32_32x32x16_bf16, the
//    group's queries held in registers (q_pe rotated once, at the query position);
//  * online softmax in the log2 domain, with the running maximum raised only when a tile
//    exceeds it by more than 2^8 (then O and l are rescaled), so most tiles rescale nothing;
//  * P leaves the score accumulator already in the layout the P · V product takes as its B
//    operand (the position order inside a K-step is permuted identically on both operands);
//    O^T [D_v x rows] += V_g^T · P^T with V_g read by transposing LDS reads;
//  * each split writes (O / l as bf16, m + log2 l) for the merge kernel, which combines the
//    splits by their log-sum-exp.
#include "common.hpp"
#include "launch.hpp"
#include "mfma_util.hpp"

namespace mla {
namespace {

using namespace mfma;

constexpr int kD = 128, kDv = 128, kDr = 64;       // per-group key, value and rotary widths
constexpr int kTok = 32;                           // positions per tile
constexpr int kKBytes = kTok * kD * 2;             // 8 KiB of K_g rows (256 B each)
constexpr int kVBytes = kTok * kDv * 2;            // 8 KiB of V_g rows (256 B each)
constexpr int kRBytes = kTok * kDr * 2;            // 4 KiB of k_r rows (128 B each)
constexpr int kSlotBytes = kKBytes + kVBytes + kRBytes;
constexpr int kSlots = 2;                          // ring slots (40 KiB: 4 workgroups per CU)
constexpr int kDmaK = kKBytes / 1024, kDmaV = kVBytes / 1024, kDmaR = kRBytes / 1024;
constexpr int kDma = kDmaK + kDmaV + kDmaR;        // 1 KiB copies per tile (20)
static_assert(kSlots >= 2 && kSlots <= 4, "ring depth the waits below cover");
constexpr int kQSteps = (kD + kDr) / 16;           // score K-steps (12)
constexpr int kDB = kDv / 32;                      // 32-wide value blocks (4)
constexpr float kLazy = 8.0f;                      // log2 headroom before the max is raised
constexpr int kMaxRows = 1 << 20;                  // query rows per group (heads x tokens)

// Physical 16-byte chunk of logical chunk c in a 256-byte row p is c ^ swz256(p): a bijection
// of p's low four bits, so 16 consecutive rows read at one logical chunk hit 16 distinct
// chunk slots, and 4 consecutive rows x 4 consecutive chunks (a transposing read of 32 lanes)
// do too. In a 128-byte row (two rows per 256 bytes) it is c ^ swz128(p).
__device__ __forceinline__ int swz256(int p) { return 4 * (p & 3) + ((p >> 2) & 3); }
__device__ __forceinline__ int swz128(int p) { return (p >> 1) & 7; }

template <int NRB>
__global__ __launch_bounds__(64) void gqa_mfma_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
    const int32_t* __restrict__ q_pos, const uint16_t* __restrict__ gqa,
    const int32_t* __restrict__ table, const int32_t* __restrict__ lens, int num_blocks,
    int max_blocks, int bs, int H, int G, int s_q, int n_split, int n_units, int n_rows,
    int nrb, int spread, float scale_log2, float lse_scale, float rope_base,
    uint16_t* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(16))) char ring[kSlots][kSlotBytes];
  // work item: blocks are handed to the 8 XCDs in turn. Without spread, the G groups of unit
  // (sequence, split), and the nrb workgroups that share a group's query rows (32 NRB rows
  // each), take consecutive turns on one XCD, where the tiles they all read stay in L2. With
  // spread (fewer units than XCDs: a prefill), the (unit, group) lines go to the XCDs in turn,
  // each line's row blocks on its XCD, the latest query rows (the longest causal range) first.
  const int id = blockIdx.x, jx = id >> 3;
  int g, rbw, unit;
  if (spread) {
    const int lj = jx / nrb;
    const int line = 8 * lj + (id & 7);
    if (line >= n_units * G) return;
    rbw = nrb - 1 - (jx - lj * nrb);
    unit = line / G;
    g = line - unit * G;
  } else {
    const int gr = jx % (G * nrb);
    g = gr / nrb;
    rbw = gr - g * nrb;
    unit = (jx / (G * nrb)) * 8 + (id & 7);
    if (unit >= n_units) return;
  }
  const int b = unit / n_split, k = unit - b * n_split;
  const int lane = threadIdx.x, l32 = lane & 31, hi = lane >> 5;
  const int hg = H / G, R = hg * s_q;
  const int capacity = max_blocks * bs;
  const int Lb = lens[b];
  const int lim_all = visible_count(Lb, s_q, s_q - 1, capacity);  // the last query sees most
  int t0, t1;
  split_range(lim_all, n_split, k, kSplitAlign, &t0, &t1);

  // rows of this lane: n = 32 (NRB rbw + rb) + l32 -> (query i, head g hg + n % hg)
  int64_t pidx[NRB];
  int lim[NRB];
  bool valid[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int n = 32 * (NRB * rbw + rb) + l32;
    valid[rb] = n < R;
    const int i = valid[rb] ? n / hg : 0;
    const int64_t qrow = (static_cast<int64_t>(b) * s_q + i) * H + g * hg + (valid[rb] ? n % hg : 0);
    pidx[rb] = static_cast<int64_t>(k) * n_rows + qrow;
    lim[rb] = valid[rb] ? visible_count(Lb, s_q, i, capacity) : 0;
  }
  {
    // the split's range ends at the workgroup's last visible position (the wave-wide maximum
    // over its rows): row blocks of early queries in a multi-token step skip later tiles
    int me = 0;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) me = max(me, lim[rb]);
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) me = max(me, __shfl_xor(me, sh, 64));
    t1 = min(t1, __builtin_amdgcn_readfirstlane(me));
  }
  const int ntiles = t1 > t0 ? cdiv(t1 - t0, kTok) : 0;

  if (ntiles == 0) {  // nothing of this split is visible: an empty partial
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      if (!valid[rb]) continue;
      if (hi == 0 && part_lse != nullptr) part_lse[pidx[rb]] = -INFINITY;
      uint4* dst = reinterpret_cast<uint4*>(part_o + pidx[rb] * kDv);
      for (int e = hi; e < kDv / 8; e += 2) dst[e] = make_uint4(0u, 0u, 0u, 0u);
    }
    return;
  }

  // copy plan of a tile: K_g and V_g copies move 4 rows x 16 chunks, k_r copies 8 rows x 8
  const int GD = G * kD, GW = G * (kD + kDv) + kDr;
  const unsigned rb_bytes = 2u * GW;
  const unsigned koff = 2u * g * kD, voff = 2u * (GD + g * kDv), roff = 2u * (GD + G * kDv);
  const int pk = lane >> 4, ck = lane & 15;   // row 4 i + pk, chunk ck of K_g / V_g copy i
  const int pr = lane >> 3, cr = lane & 7;    // row 8 i + pr, chunk cr of k_r copy i
  auto issue_tile = [&](int t, int slot) __attribute__((always_inline)) {
    const int p0 = t0 + kTok * t;
    const int jb = p0 / bs;
    int id_blk = table[static_cast<int64_t>(b) * max_blocks + jb];
    id_blk = (id_blk < 0 || id_blk >= num_blocks) ? 0 : id_blk;  // masked below, read in bounds
    const int64_t base = static_cast<int64_t>(id_blk) * bs + (p0 - jb * bs);
    const char* gbase = reinterpret_cast<const char*>(gqa) + base * rb_bytes;
    const int plim = lim_all - 1 - p0;  // rows past the end repeat the last visible row
    const unsigned lbase = lds_addr(ring[slot]);
#pragma unroll
    for (int i = 0; i < kDmaK; ++i) {
      const int p = 4 * i + pk;
      const unsigned row = static_cast<unsigned>(p < plim ? p : plim) * rb_bytes;
      const unsigned ch = 16u * (ck ^ swz256(p));
      // K_g and V_g rows are read once (one workgroup per split and group): streamed; the k_r
      // rows below, which the groups of a unit share through L2, keep the default policy
      dma16<true>(gbase, row + koff + ch, lbase + 1024 * i);
      dma16<true>(gbase, row + voff + ch, lbase + kKBytes + 1024 * i);
    }
#pragma unroll
    for (int i = 0; i < kDmaR; ++i) {
      const int p = 8 * i + pr;
      const unsigned row = static_cast<unsigned>(p < plim ? p : plim) * rb_bytes;
      dma16(gbase, row + roff + 16u * (cr ^ swz128(p)), lbase + kKBytes + kVBytes + 1024 * i);
    }
  };
#pragma unroll
  for (int i = 0; i < kSlots - 1; ++i)
    if (i < ntiles) issue_tile(i, i);

  // queries as the B operand of the scores: lane (n, hi) holds elements 16 ks + 8 hi .. +7 of
  // row n; q_pe is rotated at the query position (pairs (2j, 2j+1))
  bf16x8 qf[NRB][kQSteps];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int n = 32 * (NRB * rbw + rb) + l32;
    const int i = valid[rb] ? n / hg : 0;
    const int64_t qrow = pidx[rb] - static_cast<int64_t>(k) * n_rows;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks)
      qf[rb][ks] = valid[rb] ? *reinterpret_cast<const bf16x8*>(q_nope + qrow * kD + 16 * ks + 8 * hi)
                             : bf16x8{};
    const int pos = q_pos[static_cast<int64_t>(b) * s_q + i];
#pragma unroll
    for (int ks = 0; ks < kDr / 16; ++ks) {
      float v[8];
      if (valid[rb]) {
        const uint4 raw = *reinterpret_cast<const uint4*>(q_pe + qrow * kDr + 16 * ks + 8 * hi);
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = __uint_as_float(w4[e] << 16), x1 = __uint_as_float(w4[e] & 0xffff0000u);
          float cs, sn;
          rope_cos_sin(pos, 8 * ks + 4 * hi + e, kDr, rope_base, &cs, &sn);
          v[2 * e] = x0 * cs - x1 * sn;
          v[2 * e + 1] = x0 * sn + x1 * cs;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.f;
      }
      qf[rb][kD / 16 + ks] = to_bf16x8(v);
    }
  }

  // LDS read offsets inside a slot. Scores: row l32, logical chunk 2 ks + hi. Values
  // (transposing, 16-lane group G4, source lane 4 kk + j): row 16 s + 8 h + 4 (G4 / 2) + kk,
  // bytes 2 (32 db + 16 (G4 % 2) + 4 j) .. +7; the row's swizzle does not depend on s.
  unsigned s_off[kQSteps];
#pragma unroll
  for (int ks = 0; ks < kD / 16; ++ks) s_off[ks] = 256u * l32 + 16u * ((2 * ks + hi) ^ swz256(l32));
#pragma unroll
  for (int ks = 0; ks < kDr / 16; ++ks)
    s_off[kD / 16 + ks] = kKBytes + kVBytes + 128u * l32 + 16u * ((2 * ks + hi) ^ swz128(l32));
  const int G4 = lane >> 4, s16 = lane & 15;
  unsigned v_off[2][kDB];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 8 * h + 4 * (G4 >> 1) + (s16 >> 2);
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      const int cl = 4 * db + 2 * (G4 & 1) + ((s16 & 3) >> 1);
      v_off[h][db] = kKBytes + 256u * row + 16u * (cl ^ swz256(row)) + 8u * (s16 & 1);
    }
  }

  f32x16 o[NRB][kDB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[rb][db][r] = 0.f;
  float m_run[NRB], l_part[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) { m_run[rb] = -INFINITY; l_part[rb] = 0.f; }
  // positions from which some row of the tile is masked (a query's visible end, the split end)
  int mask_from = t1;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
    if (valid[rb]) mask_from = min(mask_from, lim[rb]);
  {
    // the wave-wide minimum over lanes
    int mf = mask_from;
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) mf = min(mf, __shfl_xor(mf, sh, 64));
    mask_from = __builtin_amdgcn_readfirstlane(mf);
  }

  for (int t = 0; t < ntiles; ++t) {
    {
      // tile t has landed when at most the copies of the tiles issued after it are in flight
      const int later = min(kSlots - 2, ntiles - 1 - t);
      if (later >= 2) wait_vm<2 * kDma>();
      else if (later == 1) wait_vm<kDma>();
      else wait_vm<0>();
    }
    // the next tile goes into the slot tile t-1 used
    if (t + kSlots - 1 < ntiles) issue_tile(t + kSlots - 1, (t + kSlots - 1) % kSlots);
    const char* slot = ring[t % kSlots];
    const int p0 = t0 + kTok * t;
    const int jb = p0 / bs;
    const int id_blk = table[static_cast<int64_t>(b) * max_blocks + jb];
    const bool tile_ok = id_blk >= 0 && id_blk < num_blocks;
    const bool masked = !tile_ok || p0 + kTok > mask_from;

    f32x16 sc[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[rb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks) {
      const bf16x8 a = lds16(slot + s_off[ks]);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        sc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[rb][ks], sc[rb], 0, 0, 0);
    }

    // register r holds position p0 + 8 (r / 4) + 4 hi + r % 4 of row 32 rb + l32
    bf16x8 pb[NRB][2];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      float s[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = sc[rb][r] * scale_log2;
      if (masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int p = p0 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (!tile_ok || p >= lim[rb] || p >= t1) s[r] = -INFINITY;
        }
      }
      float mt = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
      mt = max_xor32(mt);
      const bool raise = mt > m_run[rb] + kLazy;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float alpha =
            raise ? (m_run[rb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[rb] - mt)) : 1.f;
        if (raise) m_run[rb] = mt;
        l_part[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[rb][db][r] *= alpha;
      }
      const float mu = m_run[rb] == -INFINITY ? 0.f : m_run[rb];
      float p[16];
      float ls = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = __builtin_amdgcn_exp2f(s[r] - mu);  // exp2(-inf) = 0
        ls += p[r];
      }
      l_part[rb] += ls;
      pb[rb][0] = to_bf16x8(p);
      pb[rb][1] = to_bf16x8(p + 8);
    }

#pragma unroll
    for (int sg = 0; sg < 2; ++sg) {
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const bf16x8 va = lds_read_tr2(slot + v_off[0][db] + 4096 * sg, slot + v_off[1][db] + 4096 * sg);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          o[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[rb][sg], o[rb][db], 0, 0, 0);
      }
    }
  }

  // O^T register r of block db holds value column 32 db + 8 (r / 4) + 4 hi + r % 4 of row
  // 32 rb + l32: four consecutive columns per register quad, stored as 8 bytes
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const float l_tot = sum_xor32(l_part[rb]);
    if (!valid[rb]) continue;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (hi == 0 && part_lse != nullptr)
      part_lse[pidx[rb]] = l_tot > 0.f ? (m_run[rb] + log2f(l_tot)) * lse_scale : -INFINITY;
    uint16_t* dst = part_o + pidx[rb] * kDv;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint2*>(dst + 32 * db + 8 * q + 4 * hi) =
            make_uint2(pack_bf16x2(o[rb][db][4 * q] * inv, o[rb][db][4 * q + 1] * inv),
                       pack_bf16x2(o[rb][db][4 * q + 2] * inv, o[rb][db][4 * q + 3] * inv));
  }
}

}  // namespace

bool gqa_mfma_fits(const mla_dims& d, int s_q) {
  if (d.dtype != MLA_BF16 || (d.flags & MLA_FLAG_GENERIC_KERNELS)) return false;
  if (d.d_nope != kD || d.d_v != kDv || d.d_r != kDr || d.block_size % kTok != 0) return false;
  if (d.n_groups < 1 || d.n_heads % d.n_groups != 0) return false;
  return static_cast<int64_t>(d.n_heads / d.n_groups) * s_q <= kMaxRows;
}

hipError_t launch_gqa_mfma(const mla_dims& d, int batch, int s_q, const void* q_nope,
                           const void* q_pe, const int32_t* q_pos, const void* gqa,
                           int num_blocks, const int32_t* table, int max_blocks,
                           const int32_t* seq_lens, int n_split, void* part_o, float* part_lse,
                           bool direct, hipStream_t s) {
  const float scale_log2 = softmax_scale_of(d) * 1.4426950408889634f;
  const int n_units = batch * n_split;
  const int n_rows = batch * s_q * d.n_heads;
  const int R = (d.n_heads / d.n_groups) * s_q;
  // a group's query rows go to workgroups of 32 rows each (one row block per wave), which read
  // the same tiles through L2: at 64 rows (s_q = 4, G = 8) this measured 1.21 ms against
  // 1.35 ms for both row blocks in one wave (NRB = 2)
  // With few (sequence, split) units and many rows (a prefill, bound by the matrix cores
  // rather than HBM) each wave takes two row blocks, halving the tile copies per product.
  const int spread = n_units < 8;
  const bool two = spread && R > 64;
  const int nrb = cdiv(R, two ? 64 : 32);
  const int64_t n_wg = spread ? 8 * static_cast<int64_t>(nrb) * cdiv(n_units * d.n_groups, 8)
                              : 8 * static_cast<int64_t>(d.n_groups) * nrb * cdiv(n_units, 8);
  // direct: one split, written as the final output (O / l) and natural-log lse
  const float lse_scale = direct ? 0.6931471805599453f : 1.0f;
  if (n_wg > INT32_MAX) return hipErrorInvalidConfiguration;
#define MLA_LAUNCH(NRB_)                                                                    \
  hipLaunchKernelGGL(gqa_mfma_kernel<NRB_>, dim3(static_cast<unsigned>(n_wg)), dim3(64), 0, s, \
                     static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_pe),  \
                     q_pos, static_cast<const uint16_t*>(gqa), table, seq_lens, num_blocks,     \
                     max_blocks, d.block_size, d.n_heads, d.n_groups, s_q, n_split, n_units,    \
                     n_rows, nrb, spread, scale_log2, lse_scale, d.rope_base,                  \
                     static_cast<uint16_t*>(part_o), part_lse)
  if (two)
    MLA_LAUNCH(2);
  else
    MLA_LAUNCH(1);
#undef MLA_LAUNCH
  return hipGetLastError();
}

}  // namespace mla
