// Device helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_WAVE 64

namespace moe {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
  return v;
}

// Sum over aligned groups of LPR lanes (LPR a power of two <= 64); every lane
// of the group receives the group's sum.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
  return v;
}

// ---------------------------------------------------------------------------
// int4 decode, bf16 offset form (GEMV kernels).
//
// One 32-bit word holds 8 nibbles e0..e7 (e_i in bits 4i..4i+3, element i of
// the 8).  With the bf16 exponent of 128 (0x4300) and a nibble OR-ed into the
// low 4 of the 7 mantissa bits, a 16-bit half is exactly the bf16 value
// 128 + e.  Shifts by 0, 4, 8, 12 and a mask keeping bits 0-3 of each half
// give four bf16 pairs:
//   p0 = [128 + e0, 128 + e4]   p1 = [128 + e1, 128 + e5]
//   p2 = [128 + e2, 128 + e6]   p3 = [128 + e3, 128 + e7]
// Dotting them with activation pairs a0 = [x0, x4], a1 = [x1, x5],
// a2 = [x2, x6], a3 = [x3, x7] (products exact in fp32) gives
// sum_i (128 + e_i) x_i; subtracting the per-group constant 136 * sum_i x_i
// leaves sum_i (e_i - 8) x_i up to fp32 rounding of the sums.
// ---------------------------------------------------------------------------
struct Q4Pairs {
  uint32_t p0, p1, p2, p3;
};

__device__ __forceinline__ Q4Pairs q4_bf16_pairs(uint32_t w) {
  Q4Pairs r;
  r.p0 = (w & 0x000F000Fu) | 0x43004300u;
  r.p1 = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
  r.p2 = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
  r.p3 = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
  return r;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Pack two bf16 bit patterns into one word (lo, hi).
__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

// ---------------------------------------------------------------------------
// int4 decode, fp16 form (MFMA kernels): the MFMA operand is the exact weight
// (e - 8) * s rounded once to fp16 (nearest even).  With the fp16 exponent of
// 1024 (0x6400) the 10 mantissa bits hold a nibble either at bits 0-3 or,
// unshifted, at bits 4-7 (value 1024 + 16 e), so one shift serves two pairs:
//   [1024 + e0, 1024 + e4] - 1032            -> [e0 - 8, e4 - 8]  (exact)
//   [1024 + 16 e1, 1024 + 16 e5] / 16 - 72   -> [e1 - 8, e5 - 8]  (exact)
// then one packed multiply by [s, s] rounds the exact product.  The resulting
// fp16 vector holds the 8 elements in the order 0,4,1,5,2,6,3,7; the
// activation operands are stored in the same order (see perm8 below).
// ---------------------------------------------------------------------------
__device__ __forceinline__ f16x8_t q4_f16x8(uint32_t w, f16x2_t s2) {
  const uint32_t w8 = w >> 8;
  const f16x2_t off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const f16x2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const f16x2_t off2 = {(_Float16)-72.0f, (_Float16)-72.0f};
  f16x2_t a = __builtin_bit_cast(f16x2_t, (w & 0x000F000Fu) | 0x64006400u) + off;
  f16x2_t b = __builtin_bit_cast(f16x2_t, (w & 0x00F000F0u) | 0x64006400u) * sixteenth + off2;
  f16x2_t c = __builtin_bit_cast(f16x2_t, (w8 & 0x000F000Fu) | 0x64006400u) + off;
  f16x2_t d = __builtin_bit_cast(f16x2_t, (w8 & 0x00F000F0u) | 0x64006400u) * sixteenth + off2;
  a = a * s2;
  b = b * s2;
  c = c * s2;
  d = d * s2;
  f16x8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Position, within an aligned block of 8, at which element i is stored in the
// MFMA kernels' fp16 activation buffers (inverse of the order 0,4,1,5,2,6,3,7).
__device__ __forceinline__ int perm8_pos(int i) { return ((i & 3) << 1) | (i >> 2); }

__device__ __forceinline__ float sigmoidf_acc(float z) { return 1.0f / (1.0f + expf(-z)); }

}  // namespace moe
