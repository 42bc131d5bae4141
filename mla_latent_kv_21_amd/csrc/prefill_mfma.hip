// Prefill attention over the expanded cache on gfx950 matrix cores: bf16, D = D_v = 128,
// d_r = 64, many query rows per group (heads of one group x new tokens), in one or several
// splits of the history (the latter for multi-token decode steps).
//
// What is computed is the no-cache pass of the Smallem article ("Le code": every head's keys
// and values are key_up and value_up of the latent; "Deux produits ou une concaténation ?":
// one score product over [k_nope ; k_r] and [q_nope ; q_r]) with the causal visibility of a
// multi-token step, over the rows gqla_expand wrote ([K_0 .. K_{G-1} || V_0 .. || k_r]). With
// many query rows per group it is bound by the matrix cores, not by HBM, so unlike the decode
// kernel a tile of the cache is shared by four waves:
//
//  * one workgroup per (sequence, group, 128 query rows): four waves of 32 rows; the row
//    blocks of one (sequence, group) run on one XCD (the tiles they all read stay in L2), the
//    latest rows (the longest causal range) first;
//  * 32-position tiles of K_g (256 B), V_g (256 B) and k_r (128 B) per position (20 KiB, inside
//    one cache block) stream HBM -> LDS with global_load_lds_dwordx4 into a 3-slot ring, two
//    tiles ahead, each wave issuing a quarter of a tile's copies, one barrier per tile; 16-byte
//    chunks XOR-swizzled by position as in the decode kernel;
//  * per wave: S^T [32 positions x 32 rows] = [K_g | k_r] · Q^T on v_mfma_f32_32x32x16_bf16
//    (queries in registers, q_pe rotated once at the query position), online softmax in the
//    log2 domain with the running maximum raised only past 2^8 of headroom, P kept in the
//    score accumulator's layout as the B operand of O^T += V_g^T · P^T (V_g read by
//    transposing LDS reads); a wave skips the tiles past its rows' causal end;
//  * two workgroups per CU (registers capped at 256 per lane), so that one wave's softmax
//    overlaps the other's products on each SIMD;
//  * with one split (direct) the output O / l (bf16) and the natural-log lse are written
//    directly; with several, split k writes its normalised bf16 partial and its log2-domain
//    lse at row k * n_rows + row, the layout gqa_mfma_kernel writes, for the GQA merge.
#include <climits>
#include <type_traits>

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
constexpr int kSlots = 3;                          // ring slots (60 KiB: two workgroups per CU)
constexpr int kWaves = 4;
constexpr int kRows = 32 * kWaves;                 // query rows per workgroup
constexpr int kCopiesPerWave = kSlotBytes / 1024 / kWaves;   // 1 KiB copies per wave per tile
static_assert(kCopiesPerWave == 5, "the copy plan below: K, K, V, V, k_r");
constexpr int kQSteps = (kD + kDr) / 16;           // score K-steps (12)
constexpr int kDB = kDv / 32;                      // 32-wide value blocks (4)
constexpr float kLazy = 8.0f;                      // log2 headroom before the max is raised

// Physical 16-byte chunk of logical chunk c in a 256-byte row p is c ^ swz256(p); in a
// 128-byte row c ^ swz128(p) (conflict-free score reads and transposing value reads).
__device__ __forceinline__ int swz256(int p) { return 4 * (p & 3) + ((p >> 2) & 3); }
__device__ __forceinline__ int swz128(int p) { return (p >> 1) & 7; }

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) v = max(v, __shfl_xor(v, sh, 64));
  return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) v = min(v, __shfl_xor(v, sh, 64));
  return __builtin_amdgcn_readfirstlane(v);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_mfma_kernel(const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
                         const int32_t* __restrict__ q_pos, const uint16_t* __restrict__ gqa,
                         const int32_t* __restrict__ table, const int32_t* __restrict__ lens,
                         int num_blocks, int max_blocks, int bs, int H, int G, int s_q,
                         int batch, int n_split, int n_rows, int nrb, int spread,
                         float scale_log2, float lse_scale, float rope_base,
                         uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) char ring[kSlots][kSlotBytes];
  // work item (unit = (sequence, split), group, row block). With spread (fewer units than
  // XCDs: a prefill) the (unit, group) lines go to the 8 XCDs in turn, a line's row blocks on
  // its XCD, the last row block first; otherwise the groups and row blocks of a unit take
  // consecutive turns on one XCD, where the k_r rows they all read stay in L2.
  const int id = blockIdx.x, jx = id >> 3;
  const int n_units = batch * n_split;
  int unit, g, rbw;
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
  const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hg = H / G, R = hg * s_q;
  const int capacity = max_blocks * bs;
  const int Lb = lens[b];
  // this split's positions [t0, t1) of those the last query sees
  int t0, t1;
  split_range(visible_count(Lb, s_q, s_q - 1, capacity), n_split, k, kSplitAlign, &t0, &t1);

  // this lane's row: n = 128 rbw + 32 w + l32 -> (query i = n / hg, head g hg + n % hg)
  const int n = kRows * rbw + 32 * w + l32;
  const bool valid = n < R;
  const int i = valid ? n / hg : 0;
  const int64_t qrow = (static_cast<int64_t>(b) * s_q + i) * H + g * hg + (valid ? n % hg : 0);
  const int lim = valid ? min(visible_count(Lb, s_q, i, capacity), t1) : 0;
  // the workgroup streams positions up to its last row's end; a wave computes up to its own
  // rows' largest end and masks from their smallest
  const int n_last = min(R - 1, kRows * rbw + kRows - 1);
  const int wg_end = min(t1, max(0, visible_count(Lb, s_q, n_last / hg, capacity)));
  const int ntiles = wg_end > t0 ? cdiv(wg_end - t0, kTok) : 0;
  const int wave_end = wave_max(lim);
  const int mask_from = wave_min(valid ? lim : INT_MAX);

  // queries as the B operand of the scores: lane (n, hi) holds elements 16 ks + 8 hi .. +7 of
  // its row; q_pe rotated at the query position (pairs (2j, 2j+1))
  bf16x8 qf[kQSteps];
#pragma unroll
  for (int ks = 0; ks < kD / 16; ++ks)
    qf[ks] = valid ? *reinterpret_cast<const bf16x8*>(q_nope + qrow * kD + 16 * ks + 8 * hi)
                   : bf16x8{};
  {
    const int pos = q_pos[static_cast<int64_t>(b) * s_q + i];
#pragma unroll
    for (int ks = 0; ks < kDr / 16; ++ks) {
      float v[8];
      if (valid) {
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
      qf[kD / 16 + ks] = to_bf16x8(v);
    }
  }

  // copy plan of a tile: 20 copies of 1 KiB, copy c = w + 4 j of wave w: K_g rows 4 c + pk
  // (j = 0, 1), V_g rows 4 (c - 8) + pk (j = 2, 3), k_r rows 8 (c - 16) + pr (j = 4); chunk
  // ck (cr) of each row
  const int GD = G * kD, GW = G * (kD + kDv) + kDr;
  const unsigned rb_bytes = 2u * GW;
  const unsigned koff = 2u * g * kD, voff = 2u * (GD + g * kDv), roff = 2u * (GD + G * kDv);
  const int pk = lane >> 4, ck = lane & 15;
  const int pr = lane >> 3, cr = lane & 7;
  auto issue_tile = [&](int t, int slot) __attribute__((always_inline)) {
    const int p0 = t0 + kTok * t;
    const int jb = p0 / bs;
    int id_blk = table[static_cast<int64_t>(b) * max_blocks + jb];
    id_blk = (id_blk < 0 || id_blk >= num_blocks) ? 0 : id_blk;  // masked below, read in bounds
    const int64_t base = static_cast<int64_t>(id_blk) * bs + (p0 - jb * bs);
    const char* gbase = reinterpret_cast<const char*>(gqa) + base * rb_bytes;
    const int plim = wg_end - 1 - p0;  // rows past the end repeat the last visible row
    const unsigned lbase = lds_addr(ring[slot]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = w + 4 * j;
      const int cc = j < 2 ? c : c - 8;
      const int p = 4 * cc + pk;
      const unsigned row = static_cast<unsigned>(p < plim ? p : plim) * rb_bytes;
      dma16(gbase, row + (j < 2 ? koff : voff) + 16u * (ck ^ swz256(p)),
            lbase + (j < 2 ? 0u : static_cast<unsigned>(kKBytes)) + 1024u * cc);
    }
    {
      const int p = 8 * w + pr;
      const unsigned row = static_cast<unsigned>(p < plim ? p : plim) * rb_bytes;
      dma16(gbase, row + roff + 16u * (cr ^ swz128(p)), lbase + kKBytes + kVBytes + 1024u * w);
    }
  };
  if (ntiles > 0) issue_tile(0, 0);
  if (ntiles > 1) issue_tile(1, 1);

  // LDS read offsets inside a slot. Scores: row l32, logical chunk 2 ks + hi. Values
  // (transposing, 16-lane group G4, source lane 4 kk + j): row 16 s + 8 h + 4 (G4 / 2) + kk,
  // bytes 2 (32 db + 16 (G4 % 2) + 4 j) .. +7
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

  f32x16 o[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_run = -INFINITY, l_part = 0.f;

  // one tile of this wave's rows from the slot at `slot`
  auto tile_body = [&](const char* slot, int p0, bool tile_ok, bool masked)
                       __attribute__((always_inline)) {
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks)
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds16(slot + s_off[ks]), qf[ks], sc, 0, 0, 0);

    // register r holds position p0 + 8 (r / 4) + 4 hi + r % 4 of row l32; the scale (> 0) is
    // applied inside the exponent, so the raw scores are masked and their maximum scaled
    if (masked) {
      // (the empty asm keeps this branch a branch: speculated, it costs every tile 60 VALU)
      asm volatile("" ::: "memory");
      const int d = lim - p0 - 4 * hi;  // element r is past this row's end when its offset >= d
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (!tile_ok || 8 * (r >> 2) + (r & 3) >= d) sc[r] = -INFINITY;
      }
    }
    float mt = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sc[r]);
    mt = max_xor32(mt) * scale_log2;
    const bool raise = mt > m_run + kLazy;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float alpha =
          raise ? (m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mt)) : 1.f;
      if (raise) m_run = mt;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    const float nmu = m_run == -INFINITY ? 0.f : -m_run;
    float p[16];
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], scale_log2, nmu));  // exp2(-inf) = 0
      ls += p[r];
    }
    l_part += ls;
    const bf16x8 pb0 = to_bf16x8(p), pb1 = to_bf16x8(p + 8);
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      const bf16x8 va = lds_read_tr2(slot + v_off[0][db], slot + v_off[1][db]);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb0, o[db], 0, 0, 0);
    }
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      const bf16x8 va = lds_read_tr2(slot + v_off[0][db] + 4096, slot + v_off[1][db] + 4096);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb1, o[db], 0, 0, 0);
    }
  };

  // tile t of the loop; the loop is unrolled by the ring depth so that every slot's LDS address
  // is a constant (the operand reads then take it as an immediate offset)
  auto step = [&](int t, auto kSlot) __attribute__((always_inline)) {
    constexpr int S = decltype(kSlot)::value;
    // tile t has landed (for this wave's copies) once only tile t + 1's may be in flight
    if (t + 1 < ntiles)
      wait_vm<kCopiesPerWave>();
    else
      wait_vm<0>();
    __syncthreads();  // every wave's copies of tile t are in; tile t - 1's slot is free
    if (t + 2 < ntiles) issue_tile(t + 2, (S + 2) % kSlots);
    const int p0 = t0 + kTok * t;
    if (p0 >= wave_end) return;  // past every row of this wave (it still takes the barriers)
    const int jb = p0 / bs;
    const int id_blk = table[static_cast<int64_t>(b) * max_blocks + jb];
    const bool tile_ok = id_blk >= 0 && id_blk < num_blocks;
    tile_body(ring[S], p0, tile_ok, !tile_ok || p0 + kTok > mask_from);
  };
  static_assert(kSlots == 3, "the unrolled loop below");
  for (int t = 0; t < ntiles; t += kSlots) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>{});
    if (t + 2 < ntiles) step(t + 2, std::integral_constant<int, 2>{});
  }

  // O^T register r of block db holds value column 32 db + 8 (r / 4) + 4 hi + r % 4 of row
  // l32: four consecutive columns per register quad, stored as 8 bytes
  const float l_tot = sum_xor32(l_part);
  if (!valid) return;
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  // the row's output (one split, natural-log lse) or split k's partial (log2-sum-exp)
  const int64_t oidx = static_cast<int64_t>(k) * n_rows + qrow;
  if (hi == 0 && lse != nullptr)
    lse[oidx] = l_tot > 0.f ? (m_run + log2f(l_tot)) * lse_scale : -INFINITY;
  uint16_t* dst = out + oidx * kDv;
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint2*>(dst + 32 * db + 8 * q + 4 * hi) =
          make_uint2(pack_bf16x2(o[db][4 * q] * inv, o[db][4 * q + 1] * inv),
                     pack_bf16x2(o[db][4 * q + 2] * inv, o[db][4 * q + 3] * inv));
}

}  // namespace

bool prefill_mfma_fits(const mla_dims& d, int s_q) {
  if (d.dtype != MLA_BF16 || (d.flags & MLA_FLAG_GENERIC_KERNELS)) return false;
  if (d.d_nope != kD || d.d_v != kDv || d.d_r != kDr || d.block_size % kTok != 0) return false;
  if (d.n_groups < 1 || d.n_heads % d.n_groups != 0) return false;
  return static_cast<int64_t>(d.n_heads / d.n_groups) * s_q >= kRows / 2;
}

hipError_t launch_prefill_mfma(const mla_dims& d, int batch, int s_q, const void* q_nope,
                               const void* q_pe, const int32_t* q_pos, const void* gqa,
                               int num_blocks, const int32_t* table, int max_blocks,
                               const int32_t* seq_lens, int n_split, void* out, float* lse,
                               bool direct, hipStream_t s) {
  const float scale_log2 = softmax_scale_of(d) * 1.4426950408889634f;
  const int64_t R = static_cast<int64_t>(d.n_heads / d.n_groups) * s_q;
  const int nrb = static_cast<int>((R + kRows - 1) / kRows);
  const int n_units = batch * n_split;
  const int spread = n_units < 8;
  const int64_t n_wg = spread ? 8 * static_cast<int64_t>(nrb) * cdiv(n_units * d.n_groups, 8)
                              : 8 * static_cast<int64_t>(d.n_groups) * nrb * cdiv(n_units, 8);
  if (n_wg > INT32_MAX) return hipErrorInvalidConfiguration;
  const int n_rows = batch * s_q * d.n_heads;
  const float lse_scale = direct ? 0.6931471805599453f : 1.0f;
  hipLaunchKernelGGL(prefill_mfma_kernel, dim3(static_cast<unsigned>(n_wg)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_pe),
                     q_pos, static_cast<const uint16_t*>(gqa), table, seq_lens, num_blocks,
                     max_blocks, d.block_size, d.n_heads, d.n_groups, s_q, batch, n_split,
                     n_rows, nrb, spread, scale_log2, lse_scale, d.rope_base,
                     static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace mla
