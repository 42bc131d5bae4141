// gqla_expand: rebuild the G key groups and G value groups of every cached position once,
// [c · W_UK[:, 0..G-1] || c · W_UV[:, 0..G-1] || k_r], into the expanded GQA cache (GQLA summary,
// section 2, "Chemin GQA": the latent is expanded once, and decode then runs plain GQA with no
// expansion per step).
//
// bf16 caches whose widths are multiples of 8 (d_c of 64) run on the matrix cores
// (expand_mfma: 256 positions x 256 columns per workgroup). Everything else takes the portable
// kernel: a tiled product over 64 positions x 64 output columns per workgroup with fp32
// arithmetic, latents gathered through the block table into LDS. In both, the workgroups of
// column tile 0 also copy k_r.
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

constexpr int kXPos = 256;                      // positions per workgroup (128 per wave)
constexpr int kXCols = 256;                     // expanded columns per workgroup (128 per wave)
constexpr int kXK = 64;                         // latent rows per LDS chunk (4 K-steps of 16)
constexpr int kXARow = kXK * 2 + 16;            // staged latent row: 144 B, b128 reads spread
constexpr int kXWRow = kXCols * 2 + 64;         // staged W row: 576 B, transposing reads spread
constexpr int kXABytes = kXPos * kXARow;        // 36 KiB of latents per chunk
constexpr int kXBuf = kXABytes + kXK * kXWRow;  // + 36 KiB of W per chunk
constexpr int kXORow = 128 * 2 + 16;            // staged output row of a wave: 272 B
constexpr int kXSlots = 2 * kXBuf;              // cache slots of the tile's positions (int64)

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef float __attribute__((ext_vector_type(2))) f32x2_t;
typedef uint32_t __attribute__((ext_vector_type(4))) u32x4_t;

// two floats to bf16 (round to nearest even) in one conversion instruction
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// bf16 expansion on matrix cores. A workgroup computes 256 positions x 256 expanded columns
// over the whole latent width, in chunks of 64 latent rows that are staged, double-buffered,
// in LDS: the gathered latent rows (row-major) and the matching rows of W = [W_UK | W_UV].
// Wave w owns positions 128 (w % 2) .. +127 and columns 128 (w / 2) .. +127 as 4 x 4 blocks
// of 32 x 32. Each block is computed transposed, out^T = W^T C^T: the W fragment (matrix A)
// comes from a transposing LDS read that gives each lane 8 consecutive latent rows of one
// column, the latent fragment (matrix B) is 16 contiguous bytes of one position's row, and
// each lane ends up with 4 consecutive columns of one position per register quad, stored as
// 8 bytes. Workgroups are numbered so that the column tiles of a position tile run on one XCD
// (blocks are handed to the 8 XCDs in turn), where its latent rows stay in L2; the workgroups
// of column tile 0 also copy k_r.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void expand_mfma(const uint16_t* __restrict__ latent, int num_blocks,
                 const int32_t* __restrict__ table, int max_blocks, const int32_t* __restrict__ lens,
                 const int32_t* __restrict__ start_pos, int bs, int d_c, int d_r, int G, int D,
                 int Dv, const uint16_t* __restrict__ w_uk, const uint16_t* __restrict__ w_uv,
                 uint16_t* __restrict__ gqa, int ptiles_per_seq, int n_ptiles, int n_ctiles) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kXBuf + kXPos * 8];
  static_assert(4 * 128 * kXORow <= 2 * kXBuf, "output staging fits in the chunk buffers");
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

  // cache slot of each of the tile's positions (-1: not expanded)
  int64_t* slot_of = reinterpret_cast<int64_t*>(lds + kXSlots);
  {
    const int p = p0 + tid;
    slot_of[tid] = (p >= P0 && p < L) ? cache_slot(table, max_blocks, bs, num_blocks, b, p) : -1;
  }
  __syncthreads();
  // staging: thread tid moves 16 bytes of latent rows tid / 8 + 32 u and of W rows tid / 32 + 8 u.
  // Rows of positions that are not expanded, and columns past the end, read some valid row
  // instead (slot 0, the last 8 columns): their products are never stored.
  const int c16 = tid & 7;
  const uint16_t* asrc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t sl = slot_of[(tid >> 3) + 32 * u];
    asrc[u] = latent + (sl >= 0 ? sl * row_w : 0) + 8 * c16;
  }
  const int wcol = min(c0 + 8 * (tid & 31), ncol - 8);
  const int64_t wstride = wcol < nuk ? nuk : nuv;
  const uint16_t* wsrc = (wcol < nuk ? w_uk + wcol : w_uv + (wcol - nuk)) + (tid >> 5) * wstride;
  u32x4_t ra[8], rw[8];
  auto load_chunk = [&](int kk) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 8; ++u) ra[u] = *reinterpret_cast<const u32x4_t*>(asrc[u] + kk);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      rw[u] = *reinterpret_cast<const u32x4_t*>(wsrc + (kk + 8 * u) * wstride);
  };
  auto store_chunk = [&](char* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      *reinterpret_cast<u32x4_t*>(buf + ((tid >> 3) + 32 * u) * kXARow + 16 * c16) = ra[u];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      *reinterpret_cast<u32x4_t*>(buf + kXABytes + ((tid >> 5) + 8 * u) * kXWRow + 16 * (tid & 31)) = rw[u];
  };

  // fragment addresses: latent row 128 wp + 32 pn + l32 at K offset 8 hi; transposing W read of
  // 16-lane group G4, source lane 4 k' + j: latent row 8 (G4 / 2) + k' (+4), columns
  // 128 wc + 16 (G4 % 2) + 4 j .. +3 of the block
  const int wp = w & 1, wc = w >> 1;
  const int G4 = lane >> 4, s16 = lane & 15;
  const int a_off = (128 * wp + l32) * kXARow + 16 * hi;
  const int w_off = kXABytes + (8 * (G4 >> 1) + (s16 >> 2)) * kXWRow +
                    2 * (128 * wc + 16 * (G4 & 1) + 4 * (s16 & 3));
  // the latent fragments first: the first products of a K-step need all four of them and
  // the first W fragment
  auto read_frags = [&](const char* buf, int ks, bf16x8 (&wf)[4], bf16x8 (&cf)[4])
      __attribute__((always_inline)) {
#pragma unroll
    for (int pn = 0; pn < 4; ++pn)
      cf[pn] = *reinterpret_cast<const bf16x8*>(buf + a_off + 32 * pn * kXARow + 32 * ks);
#pragma unroll
    for (int cm = 0; cm < 4; ++cm) {
      const char* bp = buf + w_off + 16 * ks * kXWRow + 64 * cm;
      const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)((lds_char_t*)bp));
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_t*)((lds_char_t*)(bp + 4 * kXWRow)));
      wf[cm] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  f32x16 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  load_chunk(0);
  for (int kk = 0; kk < d_c; kk += kXK) {
    // chunk kk goes from registers into buffer (kk / 64) % 2, last read two chunks ago: the
    // barrier of the previous chunk has seen every wave finish that read. One barrier per chunk.
    char* cur = lds + ((kk / kXK) & 1) * kXBuf;
    store_chunk(cur);
    __syncthreads();
    // the next chunk's loads overlap this chunk's products (the last chunk reloads itself)
    load_chunk(kk + kXK < d_c ? kk + kXK : kk);
    bf16x8 wf[2][4], cf[2][4];
    read_frags(cur, 0, wf[0], cf[0]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      // fragments of the next K-step are read while this one's 16 products run
      if (ks < 3) read_frags(cur, ks + 1, wf[(ks + 1) & 1], cf[(ks + 1) & 1]);
#pragma unroll
      for (int cm = 0; cm < 4; ++cm)
#pragma unroll
        for (int pn = 0; pn < 4; ++pn)
          acc[4 * cm + pn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks & 1][cm], cf[ks & 1][pn],
                                                                      acc[4 * cm + pn], 0, 0, 0);
    }
    // order after the barrier: the next chunk's global loads, the first K-step's fragments,
    // then each K-step's products with the next K-step's reads threaded between them
    __builtin_amdgcn_sched_group_barrier(0x020, 16, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 10, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
  }

  // the accumulators go through LDS so that the stores are whole rows: wave w stages its
  // 128 x 128 outputs as bf16, position-major; register r of block (cm, pn) holds column
  // 32 cm + 8 (r / 4) + 4 hi + r % 4 of the wave's columns for position 32 pn + l32
  __syncthreads();  // every wave is done with the chunk buffers
  char* stage = lds + w * 128 * kXORow;
#pragma unroll
  for (int cm = 0; cm < 4; ++cm)
#pragma unroll
    for (int pn = 0; pn < 4; ++pn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& a = acc[4 * cm + pn];
        *reinterpret_cast<uint2*>(stage + (32 * pn + l32) * kXORow + 2 * (32 * cm + 8 * g + 4 * hi)) =
            make_uint2(pack2_bf16(a[4 * g], a[4 * g + 1]), pack2_bf16(a[4 * g + 2], a[4 * g + 3]));
      }
  __syncthreads();
  // 16 lanes per position, 16 bytes each: 4 positions per store
  const int seg = lane & 15;
  const int col = c0 + 128 * wc + 8 * seg;
  if (col < ncol) {
#pragma unroll 8
    for (int i = 0; i < 32; ++i) {
      const int row = 4 * i + (lane >> 4);
      const int64_t sl = slot_of[128 * wp + row];
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + row * kXORow + 16 * seg);
      if (sl >= 0) *reinterpret_cast<u32x4_t*>(gqa + sl * gw + col) = v;
    }
  }
  if (ct == 0) {  // k_r of each expanded position, copied as is
#pragma unroll
    for (int u = 0; u < 8; ++u) {
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
