// gqla_expand: rebuild the G key groups and G value groups of every cached position once,
// [c · W_UK[:, 0..G-1] || c · W_UV[:, 0..G-1] || k_r], into the expanded GQA cache (GQLA summary,
// section 2, "Chemin GQA": the latent is expanded once, and decode then runs plain GQA with no
// expansion per step).
//
// bf16 caches whose widths are multiples of 8 (d_c of 32) run on the matrix cores
// (expand_mfma: 128 positions x 256 columns per workgroup, two workgroups per CU). Everything
// else takes the portable kernel: a tiled product over 64 positions x 64 output columns per
// workgroup with fp32 arithmetic, latents gathered through the block table into LDS. In both,
// the workgroups of column tile 0 also copy k_r.
#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kRowT = 64, kColT = 64, kKT = 32;

template <typename T>
__global__ __launch_bounds__(256) void expand_kernel(
    const T* __restrict__ latent, int num_blocks, const int32_t* __restrict__ table,
    int max_blocks, const int32_t* __restrict__ lens, const int32_t* __restrict__ start_pos,
    int bs, int d_c, int d_r, int G, int D, int Dv, const T* __restrict__ w_uk,
    const T* __restrict__ w_uv, T* __restrict__ gqa) {
  __shared__ float cs[kRowT][kKT + 1];
  __shared__ float ws[kKT][kColT + 1];
  __shared__ int64_t slots[kRowT];
  const int b = blockIdx.y;
  const int p0 = blockIdx.x * kRowT;
  const int capacity = max_blocks * bs;
  int L = lens[b];
  L = L > capacity ? capacity : L;
  int P0 = start_pos != nullptr ? start_pos[b] : 0;
  P0 = P0 < 0 ? 0 : P0;
  if (p0 + kRowT <= P0 || p0 >= L) return;
  const int row_w = d_c + d_r;
  const int gw = G * D + G * Dv + d_r;
  for (int r = threadIdx.x; r < kRowT; r += blockDim.x) {
    const int p = p0 + r;
    slots[r] = (p >= P0 && p < L) ? cache_slot(table, max_blocks, bs, num_blocks, b, p) : -1;
  }
  __syncthreads();
  const int c0 = blockIdx.z * kColT;
  const int ncol = G * D + G * Dv;
  const int tr = (threadIdx.x >> 4) * 4, tc = (threadIdx.x & 15) * 4;
  float acc[4][4] = {};
  for (int kk = 0; kk < d_c; kk += kKT) {
    for (int e = threadIdx.x; e < kRowT * kKT; e += blockDim.x) {
      const int r = e / kKT, k = e % kKT;
      const int64_t sl = slots[r];
      cs[r][k] = (sl >= 0 && kk + k < d_c) ? ld(latent, sl * row_w + kk + k) : 0.f;
    }
    for (int e = threadIdx.x; e < kKT * kColT; e += blockDim.x) {
      const int k = e / kColT, c = e % kColT;
      const int col = c0 + c, kg = kk + k;
      float w = 0.f;
      if (kg < d_c && col < ncol) {
        w = col < G * D ? ld(w_uk, static_cast<int64_t>(kg) * (G * D) + col)
                        : ld(w_uv, static_cast<int64_t>(kg) * (G * Dv) + (col - G * D));
      }
      ws[k][c] = w;
    }
    __syncthreads();
    for (int k = 0; k < kKT; ++k) {
      float cv[4], wv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) { cv[u] = cs[tr + u][k]; wv[u] = ws[k][tc + u]; }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] += cv[u] * wv[v];
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t sl = slots[tr + u];
    if (sl < 0) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int col = c0 + tc + v;
      if (col < ncol) st(gqa, sl * gw + col, acc[u][v]);
    }
  }
  if (blockIdx.z == 0) {
    for (int e = threadIdx.x; e < kRowT * d_r; e += blockDim.x) {
      const int r = e / d_r, j = e % d_r;
      const int64_t sl = slots[r];
      if (sl >= 0) st(gqa, sl * gw + ncol + j, ld(latent, sl * row_w + d_c + j));
    }
  }
}

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef short __attribute__((ext_vector_type(4))) i16x4;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

constexpr int kXCols = 256;                     // expanded columns per workgroup (128 per wave)
constexpr int kXWRow = kXCols * 2 + 64;         // staged W row: 576 B, transposing reads spread
constexpr int kXORow = 128 * 2 + 16;            // staged output row of a wave: 272 B

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef float __attribute__((ext_vector_type(2))) f32x2_t;
typedef uint32_t __attribute__((ext_vector_type(4))) u32x4_t;

// two floats to bf16 (round to nearest even) in one conversion instruction
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// bf16 expansion on matrix cores. A workgroup computes 128 positions x 256 expanded columns
// over the whole latent width, in chunks of 32 latent rows staged, double-buffered, in LDS:
// the gathered latent rows and the matching rows of W = [W_UK | W_UV]. Wave w owns positions
// 64 (w % 2) .. +63 and columns 128 (w / 2) .. +127 as 2 x 4 blocks of 32 x 32: 128
// accumulators, so two workgroups share a CU and one wave's LDS traffic and waits overlap the
// other's products on the same SIMD.
//  * Each block is computed transposed, out^T = W^T C^T: the W fragment (matrix A) comes from
//    a transposing LDS read that gives each lane 8 consecutive latent rows of one column, the
//    latent fragment (matrix B) is 16 contiguous bytes of one position's row, and each lane
//    ends up with 4 consecutive columns of one position per register quad.
//  * A staged latent row is 64 bytes with its four 16-byte pieces XOR-swizzled by
//    (row / 4) % 4, so the staging writes (4 rows x 4 pieces per 16 lanes) and the fragment
//    reads (16 rows x one piece) touch distinct banks; W rows are padded to 576 bytes.
//  * The global loads of a chunk are issued two chunks ahead into one of two register sets.
//  * Outputs go through LDS, 32 positions of a wave at a time, as whole 256-byte row pieces.
//  * Workgroups are numbered so that the column tiles of a position tile run on one XCD
//    (blocks are handed to the 8 XCDs in turn), where its latent rows stay in L2; the
//    workgroups of column tile 0 also copy k_r.
constexpr int kXPos = 128;                       // positions per workgroup
constexpr int kXK = 32;                          // latent rows per chunk (2 K-steps)
constexpr int kXARow = kXK * 2;                  // staged latent row: 64 B, pieces swizzled
constexpr int kXABytes = kXPos * kXARow;         // 8 KiB
constexpr int kXBuf = kXABytes + kXK * kXWRow;   // + 18 KiB of W
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void expand_mfma(const uint16_t* __restrict__ latent, int num_blocks,
                  const int32_t* __restrict__ table, int max_blocks,
                  const int32_t* __restrict__ lens, const int32_t* __restrict__ start_pos,
                  int bs, int d_c, int d_r, int G, int D, int Dv,
                  const uint16_t* __restrict__ w_uk, const uint16_t* __restrict__ w_uv,
                  uint16_t* __restrict__ gqa, int ptiles_per_seq, int n_ptiles, int n_ctiles) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kXBuf + kXPos * 8];
  static_assert(4 * 32 * kXORow <= 2 * kXBuf, "half-block output staging fits");
  const int id = blockIdx.x;
  const int j = id >> 3;
  const int ct = j % n_ctiles;
  const int pt = (j / n_ctiles) * 8 + (id & 7);
  if (pt >= n_ptiles) return;
  const int b = pt / ptiles_per_seq;
  const int p0 = (pt - b * ptiles_per_seq) * kXPos;
  const int c0 = ct * kXCols;
  const int capacity = max_blocks * bs;
  int L = lens[b];
  L = L > capacity ? capacity : L;
  int P0 = start_pos != nullptr ? start_pos[b] : 0;
  P0 = P0 < 0 ? 0 : P0;
  if (p0 + kXPos <= P0 || p0 >= L) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int row_w = d_c + d_r;
  const int nuk = G * D, nuv = G * Dv, ncol = nuk + nuv;
  const int64_t gw = ncol + d_r;

  int64_t* slot_of = reinterpret_cast<int64_t*>(lds + 2 * kXBuf);
  if (tid < kXPos) {
    const int p = p0 + tid;
    slot_of[tid] = (p >= P0 && p < L) ? cache_slot(table, max_blocks, bs, num_blocks, b, p) : -1;
  }
  __syncthreads();
  // staging: thread tid moves 16 bytes of latent rows tid / 4 + 64 u (u < 2) and of W rows
  // tid / 32 + 8 u (u < 4); rows of positions that are not expanded, and columns past the end,
  // read some valid row instead (never stored)
  const int c4 = tid & 3;
  const uint16_t* asrc[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t sl = slot_of[(tid >> 2) + 64 * u];
    asrc[u] = latent + (sl >= 0 ? sl * row_w : 0) + 8 * c4;
  }
  const int wcol = min(c0 + 8 * (tid & 31), ncol - 8);
  const int64_t wstride = wcol < nuk ? nuk : nuv;
  const uint16_t* wsrc = (wcol < nuk ? w_uk + wcol : w_uv + (wcol - nuk)) + (tid >> 5) * wstride;
  // two chunks in registers ahead of the one being multiplied (sets 0 and 1, alternating)
  u32x4_t ra[2][2], rw[2][4];
  auto load_chunk = [&](int kk, u32x4_t (&ra_)[2], u32x4_t (&rw_)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) ra_[u] = *reinterpret_cast<const u32x4_t*>(asrc[u] + kk);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      rw_[u] = *reinterpret_cast<const u32x4_t*>(wsrc + (kk + 8 * u) * wstride);
  };
  auto store_chunk = [&](char* buf, const u32x4_t (&ra_)[2], const u32x4_t (&rw_)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = (tid >> 2) + 64 * u;
      *reinterpret_cast<u32x4_t*>(buf + row * kXARow + 16 * (c4 ^ ((row >> 2) & 3))) = ra_[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<u32x4_t*>(buf + kXABytes + ((tid >> 5) + 8 * u) * kXWRow + 16 * (tid & 31)) = rw_[u];
  };
  const int wp = w & 1, wc = w >> 1;
  const int G4 = lane >> 4, s16 = lane & 15;
  // row 64 wp + 32 pn + l32 keeps the swizzle of l32: piece (2 ks + hi) ^ ((l32 / 4) % 4)
  const int a_off = (64 * wp + l32) * kXARow;
  const int a_piece[2] = {16 * ((0 + hi) ^ ((l32 >> 2) & 3)), 16 * ((2 + hi) ^ ((l32 >> 2) & 3))};
  const int w_off = kXABytes + (8 * (G4 >> 1) + (s16 >> 2)) * kXWRow +
                    2 * (128 * wc + 16 * (G4 & 1) + 4 * (s16 & 3));
  auto read_frags = [&](const char* buf, int ks, bf16x8 (&wf)[4], bf16x8 (&cf)[2])
      __attribute__((always_inline)) {
#pragma unroll
    for (int pn = 0; pn < 2; ++pn)
      cf[pn] = *reinterpret_cast<const bf16x8*>(buf + a_off + 32 * pn * kXARow + a_piece[ks]);
#pragma unroll
    for (int cm = 0; cm < 4; ++cm) {
      const char* bp = buf + w_off + 16 * ks * kXWRow + 64 * cm;
      const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)((lds_char_t*)bp));
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_t*)((lds_char_t*)(bp + 4 * kXWRow)));
      wf[cm] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  // chunk kk: stored from its register set into buffer (kk / 32) % 2 (last read two chunks
  // ago, behind the previous chunk's barrier), then the set is refilled with chunk kk + 64 (the
  // last chunks reload themselves)
  auto chunk = [&](int kk, u32x4_t (&ra_)[2], u32x4_t (&rw_)[4]) __attribute__((always_inline)) {
    char* cur = lds + ((kk / kXK) & 1) * kXBuf;
    __builtin_amdgcn_sched_barrier(0);
    store_chunk(cur, ra_, rw_);
    __syncthreads();
    load_chunk(kk + 2 * kXK < d_c ? kk + 2 * kXK : kk, ra_, rw_);
    bf16x8 wf[2][4], cf[2][2];
    read_frags(cur, 0, wf[0], cf[0]);
    read_frags(cur, 1, wf[1], cf[1]);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int cm = 0; cm < 4; ++cm)
#pragma unroll
        for (int pn = 0; pn < 2; ++pn)
          acc[2 * cm + pn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks][cm], cf[ks][pn],
                                                                      acc[2 * cm + pn], 0, 0, 0);
  };
  // The loop body has no branch: the compiler then knows at every store which loads are still
  // in flight and waits only for the older register set (with a conditional second chunk in
  // the body its waits at the loop head drained both sets, every other chunk). The scheduling
  // barrier at the head of each chunk keeps one chunk's stores, and their waits, from being
  // hoisted into the chunk before.
  load_chunk(0, ra[0], rw[0]);
  load_chunk(kXK < d_c ? kXK : 0, ra[1], rw[1]);
  int kk = 0;
  for (; kk + 2 * kXK <= d_c; kk += 2 * kXK) {
    chunk(kk, ra[0], rw[0]);
    chunk(kk + kXK, ra[1], rw[1]);
  }
  if (kk < d_c) chunk(kk, ra[0], rw[0]);

  // outputs through LDS, 32 positions of each wave at a time, as whole 256-byte row pieces;
  // streaming (non-temporal) stores, so that the 4.4 GB of expanded rows do not push out of
  // L2 the latent rows and W that the position tile's other column tiles still read
  __syncthreads();  // every wave is done with the chunk buffers
  {
    char* stage = lds + w * 32 * kXORow;
    const int seg = lane & 15;
    const int col = c0 + 128 * wc + 8 * seg;
#pragma unroll
    for (int pn = 0; pn < 2; ++pn) {
#pragma unroll
      for (int cm = 0; cm < 4; ++cm)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& a = acc[2 * cm + pn];
          *reinterpret_cast<uint2*>(stage + l32 * kXORow + 2 * (32 * cm + 8 * g + 4 * hi)) =
              make_uint2(pack2_bf16(a[4 * g], a[4 * g + 1]), pack2_bf16(a[4 * g + 2], a[4 * g + 3]));
        }
      // a wave's LDS accesses complete in order: its rows are in place for its reads
      if (col < ncol) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = 4 * i + (lane >> 4);
          const int64_t sl = slot_of[64 * wp + 32 * pn + row];
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + row * kXORow + 16 * seg);
          if (sl >= 0) __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(gqa + sl * gw + col));
        }
      }
    }
  }
  if (ct == 0) {  // k_r of each expanded position, copied as is
    const int c16 = tid & 7;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t sl = slot_of[(tid >> 3) + 32 * u];
      if (sl < 0) continue;
      for (int q = c16; q < d_r / 8; q += 8)
        *reinterpret_cast<u32x4_t*>(gqa + sl * gw + ncol + 8 * q) =
            *reinterpret_cast<const u32x4_t*>(latent + sl * row_w + d_c + 8 * q);
    }
  }
}

}  // namespace

hipError_t launch_expand(const mla_dims& d, int batch, const void* cache, int num_blocks,
                         const int32_t* table, int max_blocks, const int32_t* seq_lens,
                         const int32_t* start_pos, const void* w_uk, const void* w_uv,
                         void* gqa, hipStream_t s) {
  const int ncol = d.n_groups * (d.d_nope + d.d_v);
  const int ptiles_per_seq = cdiv(max_blocks * d.block_size, kXPos);
  const int64_t n_ptiles64 = static_cast<int64_t>(batch) * ptiles_per_seq;
  const int64_t n_wg = 8 * static_cast<int64_t>(cdiv(ncol, kXCols)) * ((n_ptiles64 + 7) / 8);
  if (d.dtype == MLA_BF16 && !(d.flags & MLA_FLAG_GENERIC_KERNELS) && d.d_c % kXK == 0 &&
      d.d_r % 8 == 0 && (d.n_groups * d.d_nope) % 8 == 0 && (d.n_groups * d.d_v) % 8 == 0 &&
      n_wg <= INT32_MAX) {
    const int n_ptiles = static_cast<int>(n_ptiles64), n_ctiles = cdiv(ncol, kXCols);
    const dim3 xgrid(static_cast<unsigned>(n_wg));
    hipLaunchKernelGGL(expand_mfma, xgrid, dim3(256), 0, s, static_cast<const uint16_t*>(cache),
                       num_blocks, table, max_blocks, seq_lens, start_pos, d.block_size, d.d_c,
                       d.d_r, d.n_groups, d.d_nope, d.d_v, static_cast<const uint16_t*>(w_uk),
                       static_cast<const uint16_t*>(w_uv), static_cast<uint16_t*>(gqa),
                       ptiles_per_seq, n_ptiles, n_ctiles);
    return hipGetLastError();
  }
  const dim3 grid(cdiv(max_blocks * d.block_size, kRowT), batch, cdiv(ncol, kColT));
  if (d.dtype == MLA_BF16) {
    hipLaunchKernelGGL(expand_kernel<bf16>, grid, dim3(256), 0, s, static_cast<const bf16*>(cache),
                       num_blocks, table, max_blocks, seq_lens, start_pos, d.block_size, d.d_c,
                       d.d_r, d.n_groups, d.d_nope, d.d_v, static_cast<const bf16*>(w_uk),
                       static_cast<const bf16*>(w_uv), static_cast<bf16*>(gqa));
  } else {
    hipLaunchKernelGGL(expand_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(cache), num_blocks, table, max_blocks, seq_lens,
                       start_pos, d.block_size, d.d_c, d.d_r, d.n_groups, d.d_nope, d.d_v,
                       static_cast<const float*>(w_uk), static_cast<const float*>(w_uv),
                       static_cast<float*>(gqa));
  }
  return hipGetLastError();
}

}  // namespace mla
