// Small gfx950 building blocks shared by the matrix-core kernels: operand vector types, the
// global -> LDS copy, LDS addresses and transposing reads, vmcnt waits, bf16 packing and a
// lane-pair max.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {
namespace mfma {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef short __attribute__((ext_vector_type(4))) i16x4;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// One 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4): lane i's 16 bytes from
// gbase + off land at LDS byte address lds + 16 i. Issued from asm so that the compiler does
// not order LDS reads of other buffers behind it; the caller waits for these copies itself
// (vmcnt) before reading what they wrote. M0 is declared clobbered rather than saved and
// restored (two scalar instructions fewer per copy): the compiler sets it again wherever it
// needs it. kStream: the copy carries the non-temporal hint, for data that one workgroup reads
// once (a streamed cache tile), so that it does not displace what other workgroups share.
template <bool kStream = false>
__device__ __forceinline__ void dma16(const char* gbase, unsigned off, unsigned lds) {
  if constexpr (kStream) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt"
        :
        : "s"(lds), "v"(off), "s"(gbase)
        : "memory", "m0");
  } else {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2"
        :
        : "s"(lds), "v"(off), "s"(gbase)
        : "memory", "m0");
  }
}

__device__ __forceinline__ unsigned lds_addr(const char* p) {
  return static_cast<unsigned>(reinterpret_cast<size_t>((lds_char_t*)p));
}

// s_waitcnt immediate that waits for vmcnt <= n only (expcnt and lgkmcnt at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait until at most `later` vector-memory operations of this wave are still in flight: they
// complete in issue order, so everything issued before them has landed.
template <int kLater>
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLater)); }

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane i receives
// element (i % 4) of the 8 bytes addressed by lanes 4k + i/4, for k = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)((lds_char_t*)p));
}

// Two transposing reads joined into one 8-element operand: the first gives elements 0..3.
__device__ __forceinline__ bf16x8 lds_read_tr2(const char* p0, const char* p1) {
  const i16x4 a = lds_read_tr(p0), b = lds_read_tr(p1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
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

// eight floats as one bf16 operand
__device__ __forceinline__ bf16x8 to_bf16x8(const float* v) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                   pack_bf16x2(v[6], v[7])};
  return __builtin_bit_cast(bf16x8, w);
}

// max over the lane pair (lane, lane ^ 32), without going through LDS
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// sum over the lane pair (lane, lane ^ 32)
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace mfma
}  // namespace mla
