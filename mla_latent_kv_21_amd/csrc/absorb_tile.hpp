// The matrix-core tile of mla_absorb_q, shared by its own kernel and by the fused
// append-and-absorb kernel of the decode step: q_abs for one (head, 32 query rows, 128 latent
// columns) tile (Smallem article 13, "Ce que DeepSeek fait de plus": the query is carried into
// latent space once per token, q_lat = q_nope · W_UK[:, g(h)]^T; GQLA summary, section 2:
// W_UK indexed by group), plus a share of the rotary part of the tile's rows.
#pragma once

#include "common.hpp"

namespace mla {

struct AbsorbArgs {
  const uint16_t* q_nope;
  const uint16_t* q_pe;
  const int32_t* q_pos;     // [M] query positions, or NULL: row m = b s_q + i is at
  const int32_t* lens;      // position lens[b] - s_q + i (a decode step's new tokens)
  int s_q;
  const uint16_t* w_uk;
  int M, H, G, D, d_c, d_r;
  float base;
  uint16_t* q_abs;
};

// Tiles of one absorb launch: heads x row blocks of 32 x groups of four 32-column blocks.
inline int absorb_tiles(const AbsorbArgs& a, int* rblocks, int* zblocks) {
  *rblocks = cdiv(a.M, 32);
  *zblocks = cdiv(a.d_c / 32, 4);
  return a.H * *rblocks * *zblocks;
}

// Whether the matrix-core tile handles these dims, and the tile arguments of a call with M
// query rows (both defined in absorb.hip).
bool absorb_mfma_fits(const mla_dims& d);
AbsorbArgs absorb_args(const mla_dims& d, int M, const void* q_nope, const void* q_pe,
                       const int32_t* q_pos, const void* w_uk, void* q_abs);

namespace absorb_detail {
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
}  // namespace absorb_detail

// bf16 absorption on matrix cores: per head, Q_lat[32 rows x d_c] = q_nope[32 x D] ·
// W_UK[:, g]^T, i.e. a product whose operands are both contiguous along the contraction
// (rows of q_nope and rows of W_UK), so MFMA fragments load straight from memory. Tile
// (h, 32 rows from m0, column blocks 4 z .. 4 z + 3); wave w computes one 32-column block.
// The rotary (row, pair) items of the head's 32 rows are shared out over its z tiles.
// kKS: the most K-steps (D / 16) the tile is built for, 8 (D <= 128) or 16 (D <= 256): the
// fragments of both operands take 8 kKS registers, so the smaller build keeps more waves
// resident. Needs blockDim.x == 256, d_c % 32 == 0, D % 16 == 0, D <= 16 kKS.
template <int kKS>
__device__ inline void absorb_tile_mfma(const AbsorbArgs& q, int h, int m0, int z, int nz) {
  using namespace absorb_detail;
  const uint16_t* __restrict__ q_nope = q.q_nope;
  const uint16_t* __restrict__ q_pe = q.q_pe;
  const int32_t* __restrict__ q_pos = q.q_pos;
  const uint16_t* __restrict__ w_uk = q.w_uk;
  uint16_t* __restrict__ q_abs = q.q_abs;
  const int M = q.M, H = q.H, G = q.G, D = q.D, d_c = q.d_c, d_r = q.d_r;
  const float base = q.base;
  const int g = h / (H / G);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int row = d_c + d_r;
  const int ksteps = D / 16;  // at most kKS
  const int m = m0 + l32;
  bf16x8 af[kKS];
  const bf16x8 zero = {};
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    af[ks] = zero;
    if (ks < ksteps && m < M)
      af[ks] = *reinterpret_cast<const bf16x8*>(q_nope + (static_cast<int64_t>(m) * H + h) * D +
                                                16 * ks + 8 * hi);
  }
  const int64_t ldw = static_cast<int64_t>(G) * D;
  // B fragments of one 32-column block: all requested before the first MFMA
  bf16x8 bv[kKS];
  auto load_b = [&](int nb) __attribute__((always_inline)) {
    const uint16_t* wr = w_uk + (nb * 32 + l32) * ldw + static_cast<int64_t>(g) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      bv[ks] = ks < ksteps ? *reinterpret_cast<const bf16x8*>(wr + 16 * ks) : zero;
  };
  int nb = 4 * z + w;
  const int nb_end = min(d_c / 32, 4 * z + 4);
  if (nb < nb_end) load_b(nb);

  // rotary part, while the first block's fragments are in flight
  const int half = d_r / 2;
  for (int e = threadIdx.x + z * 256; e < 32 * half; e += 256 * nz) {
    const int r = e / half, jj = e % half;
    const int mm = m0 + r;
    if (mm >= M) continue;
    float cs, sn;
    const int qp = q_pos != nullptr ? q_pos[mm] : q.lens[mm / q.s_q] - q.s_q + mm % q.s_q;
    rope_cos_sin(qp, jj, d_r, base, &cs, &sn);
    const int64_t src = (static_cast<int64_t>(mm) * H + h) * d_r + 2 * jj;
    const float x0 = bf16_to_f32(q_pe[src]), x1 = bf16_to_f32(q_pe[src + 1]);
    const int64_t dst = (static_cast<int64_t>(mm) * H + h) * row + d_c + 2 * jj;
    q_abs[dst] = f32_to_bf16(x0 * cs - x1 * sn);
    q_abs[dst + 1] = f32_to_bf16(x0 * sn + x1 * cs);
  }

  while (nb < nb_end) {
    const int j = nb * 32 + l32;
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      if (ks < ksteps) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], bv[ks], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int mm = m0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (mm < M) q_abs[(static_cast<int64_t>(mm) * H + h) * row + j] = f32_to_bf16(acc[r]);
    }
    nb += 4;
    if (nb < nb_end) load_b(nb);
  }
}

}  // namespace mla
