// Device helpers shared by the MFMA attention kernels of libqsa (gfx950).
#pragma once

#include <type_traits>

#include "qsa_common.h"
#include "qsa_weights.h"

namespace qsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// Workgroup barrier that orders LDS only: it waits for this wave's LDS operations but not for
// its outstanding global loads.  (__syncthreads() also drains every global load, which would
// serialise LDS-direct prefetches issued further ahead; those are waited for with explicit
// vmcnt waits before this barrier.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }


__device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

// 16x16x32 bf16 MMA (the row sums of a P^T operand against a 0/1 selector)
__device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

// 32x32x64 8-bit MMA: A in OCP fp8 e4m3, B in e4m3 (fmt_b = 0) or bf8 e5m2 (fmt_b = 1).
template <int FMT_B>
__device__ __forceinline__ f32x16 mma8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, FMT_B, 0, 0, 0, 0);
}

// Round-to-nearest-even pack of two floats into two bf16 (low = a).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// acc + the two bf16 of p (v_dot2_f32_bf16 against (1, 1)).
__device__ __forceinline__ float dot2_ones(uint32_t p, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p), one, acc, false);
}

// max / min / sum of a value held by lane l and lane l ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(fbits(x), fbits(x), false, false);
  return fmaxf(bitsf(r[0]), bitsf(r[1]));
}
__device__ __forceinline__ float half_min(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(fbits(x), fbits(x), false, false);
  return fminf(bitsf(r[0]), bitsf(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(fbits(x), fbits(x), false, false);
  return bitsf(r[0]) + bitsf(r[1]);
}

// Key of accumulator register r of lane half hh in a 32x32 S^T block.
__device__ __forceinline__ int acc_key(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

// Two bf16 weights 2^-e0, 2^-e1 (e clipped to L-1) from t = 2^24 - y (rounded).
// bits(t) = 0x4B800000 - e; the clip is an integer max in 32 bits (so any y is
// clipped correctly), after which the low halves are -e as int16 and one
// v_pk_mad_u16 turns the pair into the bf16 exponent fields (127 - e) << 7.
__device__ __forceinline__ uint32_t pot_pair(float t0, float t1, int32_t lo) {
  const uint32_t b0 = (uint32_t)max((int32_t)fbits(t0), lo), b1 = (uint32_t)max((int32_t)fbits(t1), lo);
  const uint32_t ne = __builtin_amdgcn_perm(b1, b0, 0x05040100u);
  uint32_t w;
  asm("v_pk_mad_u16 %0, %1, %2, %3" : "=v"(w) : "v"(ne), "v"(0x00800080u), "v"(0x3F803F80u));
  return w;
}

// The same pair from t = 1 - k 2^-24 in [1/2, 1], k = (L-1) - e: the FMA that forms t with
// its output clamp to [0, 1] (v_fma_f32 ... clamp) has already clipped e to L-1 (k >= 0), and
// bits(t) = 0x3F800000 - k, so the low halves are -k as int16.  (-k)(-128) + (128 - L) 128 =
// (127 - e) 128 in each half; add holds (128 - L) 128 twice.
__device__ __forceinline__ uint32_t pot_pair_k(float t0, float t1, uint32_t add) {
  const uint32_t nk = __builtin_amdgcn_perm(fbits(t1), fbits(t0), 0x05040100u);
  uint32_t w;
  asm("v_pk_mad_u16 %0, %1, %2, %3" : "=v"(w) : "v"(nk), "v"(0xFF80FF80u), "v"(add));
  return w;
}

// t = 1 - ((L-1) - y) 2^-24 for y = -x c, rounded once and clamped to [0, 1] by one FMA: the
// rounding takes k = (L-1) - y to an integer (the ulp of [1/2, 1) is 2^-24) and the clamp at 1
// is the clip y <= L-1.  nc = -c 2^-24 and b = 1 - (L-1) 2^-24 are exact.
__device__ __forceinline__ float pot_t_clamped(float x, float nc, float b) {
  return __builtin_amdgcn_fmed3f(fmaf(x, nc, b), 0.0f, 1.0f);
}

}  // namespace qsa
