// Device helpers shared by the HIP kernels of libmla (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

// bf16 is carried as its 16 raw bits; the arithmetic is always fp32.
struct bf16 {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct Elt;
template <> struct Elt<float> {
  __device__ static __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  __device__ static __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elt<bf16> {
  __device__ static __forceinline__ float load(const bf16* p, int64_t i) {
    return bf16_to_f32(p[i].bits);
  }
  __device__ static __forceinline__ void store(bf16* p, int64_t i, float v) {
    p[i].bits = f32_to_bf16(v);
  }
};

template <typename T> __device__ __forceinline__ float ld(const T* p, int64_t i) {
  return Elt<T>::load(p, i);
}
template <typename T> __device__ __forceinline__ void st(T* p, int64_t i, float v) {
  Elt<T>::store(p, i, v);
}

// Wave64 butterfly reductions through DPP-free shuffles (ds_swizzle/bpermute chosen by the
// compiler).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide reductions for blockDim.x a multiple of 64 (<= 1024); `red` holds 16 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int i = 0; i < nw; ++i) t = fmaxf(t, red[i]);
  return t;
}

// Rotation of pair j of a d-wide rotary vector at position pos: angle pos * base^(-2j/d),
// formed and reduced in double precision so long positions keep full fp32 accuracy.
__device__ __forceinline__ void rope_cos_sin(int pos, int j, int d, float base, float* c,
                                             float* s) {
  // theta_j = base^(-2j/d) and the angle pos * theta_j in double (at position 131,071 an fp32
  // angle would be off by ~1e-2 rad); the angle is reduced to [-pi, pi] in double, and the
  // single-precision sine and cosine of the reduced angle are within ~1e-7 of the exact ones.
  const double theta = exp2(-2.0 * j / static_cast<double>(d) * log2(static_cast<double>(base)));
  const double ang = static_cast<double>(pos) * theta;
  const double kTwoPi = 6.283185307179586;
  const double red = ang - rint(ang * (1.0 / kTwoPi)) * kTwoPi;
  sincosf(static_cast<float>(red), s, c);
}

// Rotation of one rotary pair (a, q) by (cs, sn): (a cs - q sn, a sn + q cs), written with
// explicit fused multiply-adds so that every kernel that forms a cache row rounds it alike.
__device__ __forceinline__ void rope_rotate(float a, float q, float cs, float sn, float* u,
                                            float* v) {
  *u = fmaf(a, cs, -(q * sn));
  *v = fmaf(a, sn, q * cs);
}

// y * y rounded on its own (never fused into the add that follows it).
__device__ __forceinline__ float square_rn(float y) { return fmaf(y, y, 0.0f); }

// e4m3 rows. A row is stored as OCP FP8 E4M3 bytes (1 sign, 4 exponent bits of bias 7,
// 3 mantissa bits; largest finite 448, smallest subnormal 2^-9) times one fp32 scale per
// position: the smallest power of two s with amax <= 448 s (s = 1 for an all-zero row), so
// every value x / s is exact in fp32 and rounds (to nearest, ties to even) into the format's
// finite range, and byte x s is exact in bf16.
__device__ __forceinline__ int e4m3_scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int k;
  const float m = frexpf(amax, &k);  // amax = m 2^k, m in [0.5, 1)
  return m <= 0.875f ? k - 9 : k - 8;
}

// four values (already divided by the scale) as four e4m3 bytes, element 0 in the low byte
__device__ __forceinline__ unsigned e4m3_pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<unsigned>(w);
}

// Slot of position p of sequence b, or -1 when the table does not hold it in bounds.
__device__ __forceinline__ int64_t cache_slot(const int32_t* table, int max_blocks, int bs,
                                              int num_blocks, int b, int p) {
  if (p < 0) return -1;
  const int jb = p / bs;
  if (jb >= max_blocks) return -1;
  const int id = table[static_cast<int64_t>(b) * max_blocks + jb];
  if (id < 0 || id >= num_blocks) return -1;
  return static_cast<int64_t>(id) * bs + (p - jb * bs);
}

__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// Positions query i of a step may see: L - s_q + i + 1, clamped to what the table can hold.
__device__ __forceinline__ int visible_count(int L, int s_q, int i, int capacity) {
  int lim = L - s_q + i + 1;
  lim = lim > capacity ? capacity : lim;
  return lim < 0 ? 0 : lim;
}

// Split k of n_split over [0, lim): chunks of ceil(lim / n_split) rounded up to `align`
// positions; trailing splits may be empty.
__device__ __forceinline__ void split_range(int lim, int n_split, int k, int align, int* t0,
                                            int* t1) {
  const int chunk = cdiv(cdiv(lim, n_split), align) * align;
  const long long a = static_cast<long long>(k) * chunk;
  *t0 = a < lim ? static_cast<int>(a) : lim;
  *t1 = *t0 + chunk < lim ? *t0 + chunk : lim;
}

}  // namespace mla
