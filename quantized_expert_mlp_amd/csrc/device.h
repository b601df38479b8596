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

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

// 16-byte load with the nontemporal hint (streamed weights: read once).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// 16-byte load from global memory, for a pointer the compiler cannot prove
// global (one picked from an array of planes): a generic (flat) load would
// make the compiler's wait counting fall back to waiting for every
// outstanding load.
typedef __attribute__((address_space(1))) const u32x4_t global_u32x4_t;
__device__ __forceinline__ u32x4_t load_global16(const void* p) {
  return *(global_u32x4_t*)(p);
}

// Wave-uniform scalar loads (s_load, counted apart from the vector loads):
// the address must be the same in every lane, which readfirstlane makes
// explicit.  For words the kernel reads but does not write.
typedef __attribute__((address_space(4))) const int32_t const_i32_t;
typedef __attribute__((address_space(4))) const float const_f32_t;
// readfirstlane of a 64-bit address, as two 32-bit halves; the builtin
// returns int, so each half is taken back as uint32_t before widening (a
// sign-extended low half would corrupt the upper word of the address).
__device__ __forceinline__ uint64_t uniform_address(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (uint64_t)lo | ((uint64_t)hi << 32);
}
__device__ __forceinline__ int32_t load_uniform_i32(const int32_t* p) {
  return *(const_i32_t*)(uniform_address(p));
}
__device__ __forceinline__ float load_uniform_f32(const float* p) {
  return *(const_f32_t*)(uniform_address(p));
}

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

// Make LDS stores of some lanes of this wave visible to loads of other lanes
// of the same wave (LDS operations of one wave execute in order; the fences
// and the wave barrier keep the compiler from reordering or dropping the
// cross-lane accesses).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// DPP lane permutations (gfx9 encodings) used by the reductions below.  All
// of them stay inside a 16-lane DPP row, so every lane reads a live source.
enum : int {
  kDppXor1 = 0xB1,        // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,        // quad_perm [2,3,0,1]
  kDppHalfMirror = 0x141, // lane i <-> 7-i inside each half row
  kDppMirror = 0x140,     // lane i <-> 15-i inside each row
  kDppBcast15 = 0x142,    // lane 15 of row r -> every lane of row r+1
  kDppBcast31 = 0x143,    // lane 31 -> every lane of rows 2 and 3
};

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// Sum over aligned groups of LPR lanes (LPR a power of two, 4 <= LPR <= 64)
// with DPP adds.  The group's sum is valid in its last lane (kl == LPR - 1);
// for LPR <= 16 every lane of the group holds it.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(LPR >= 4 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "LPR");
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  if (LPR >= 8) v += dpp<kDppHalfMirror>(v);
  if (LPR >= 16) v += dpp<kDppMirror>(v);
  if (LPR >= 32) v += dpp<kDppBcast15, 0xA>(v);  // rows 1, 3 += row 0, 2
  if (LPR >= 64) v += dpp<kDppBcast31, 0x8>(v);  // row 3 += rows 0-1
  return v;
}

// ---------------------------------------------------------------------------
// int4 decode, bf16 offset form (GEMV kernels).
//
// One 32-bit word holds 8 nibbles e0..e7 (e_i in bits 4i..4i+3, element i of
// the 8).  t = w & 0x0F0F0F0F holds bytes [e0, e2, e4, e6] and
// u = (w >> 4) & 0x0F0F0F0F holds [e1, e3, e5, e7]; one v_perm_b32 per pair
// then interleaves two nibble bytes with the byte 0x43, giving 16-bit halves
// 0x43 0e = the exact bf16 value 128 + e (exponent of 128, the nibble in the
// low mantissa bits):
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

// v_perm_b32 selectors: byte k of the result takes byte sel_k of the pair
// (src0 = bytes 4..7, src1 = bytes 0..3).
constexpr uint32_t kSelLo = 0x04020400u;  // [src1.b0, src0.b0, src1.b2, src0.b0]
constexpr uint32_t kSelHi = 0x04030401u;  // [src1.b1, src0.b0, src1.b3, src0.b0]

__device__ __forceinline__ Q4Pairs q4_pairs_with(uint32_t w, uint32_t magic) {
  const uint32_t t = w & 0x0F0F0F0Fu;
  const uint32_t u = (w >> 4) & 0x0F0F0F0Fu;
  Q4Pairs r;
  r.p0 = __builtin_amdgcn_perm(magic, t, kSelLo);
  r.p1 = __builtin_amdgcn_perm(magic, u, kSelLo);
  r.p2 = __builtin_amdgcn_perm(magic, t, kSelHi);
  r.p3 = __builtin_amdgcn_perm(magic, u, kSelHi);
  return r;
}

__device__ __forceinline__ Q4Pairs q4_bf16_pairs(uint32_t w) { return q4_pairs_with(w, 0x43434343u); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Pack two bf16 bit patterns into one word (lo, hi).
__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

// ---------------------------------------------------------------------------
// int4 decode, fp16 form (MFMA kernels): the MFMA operand is the exact weight
// (e - 8) * s rounded once to fp16 (nearest even).  The same byte interleave
// with 0x64 gives 16-bit halves 0x64 0e = the exact fp16 value 1024 + e; one
// packed subtract of 1032 leaves e - 8 exactly, and one packed multiply by
// [s, s] rounds the exact product.  The fp16 vector holds the 8 elements in
// the order 0,4,1,5,2,6,3,7; the activation operands are stored in the same
// order (see perm8_pos below).
// ---------------------------------------------------------------------------
__device__ __forceinline__ f16x8_t q4_f16x8(uint32_t w, f16x2_t s2) {
  const Q4Pairs p = q4_pairs_with(w, 0x64646464u);
  const f16x2_t off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const f16x2_t a = (__builtin_bit_cast(f16x2_t, p.p0) + off) * s2;
  const f16x2_t b = (__builtin_bit_cast(f16x2_t, p.p1) + off) * s2;
  const f16x2_t c = (__builtin_bit_cast(f16x2_t, p.p2) + off) * s2;
  const f16x2_t d = (__builtin_bit_cast(f16x2_t, p.p3) + off) * s2;
  f16x8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// ---------------------------------------------------------------------------
// MXFP4 decode, fp16 form (MFMA kernels).  The nibbles are e2m1 codes (bit 3
// sign, bits 2..1 exponent with bias 1, bit 0 mantissa) whose eight
// magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 are fp16 values with a zero low
// byte.  One v_perm_b32 looks up the high bytes of four codes at once (its
// byte selectors 0..7 index the 8-byte table below), the sign bit moves to
// bit 7 of each byte, and the same pairing as the int4 decode spreads the
// high bytes into fp16 pairs [e0,e4], [e1,e5], [e2,e6], [e3,e7].  One packed
// multiply by the group scale [s, s] rounds the exact product once, so the
// vector holds the 8 elements in the order 0,4,1,5,2,6,3,7 like q4_f16x8.
// ---------------------------------------------------------------------------
constexpr uint32_t kE2m1Lo = 0x3E3C3800u;  // fp16 high bytes of codes 3, 2, 1, 0
constexpr uint32_t kE2m1Hi = 0x46444240u;  // codes 7, 6, 5, 4
constexpr uint32_t kSelPairLo = 0x02040004u;  // [0, b0, 0, b2] (src0 = 0 gives the zero bytes)
constexpr uint32_t kSelPairHi = 0x03040104u;  // [0, b1, 0, b3]

// fp16 high bytes of the 8 codes of one packed word: ht for the even
// elements e0, e2, e4, e6 (low nibbles), hu for the odd ones (high nibbles).
// The odd codes' sign bits already sit at bit 7 of each byte of w; the even
// codes' sit four bits lower.
struct E2m1Hi {
  uint32_t ht, hu;
};
__device__ __forceinline__ E2m1Hi e2m1_hi_bytes(uint32_t w) {
  E2m1Hi r;
  r.ht = __builtin_amdgcn_perm(kE2m1Hi, kE2m1Lo, w & 0x07070707u) | ((w << 4) & 0x80808080u);
  r.hu = __builtin_amdgcn_perm(kE2m1Hi, kE2m1Lo, (w >> 4) & 0x07070707u) | (w & 0x80808080u);
  return r;
}

__device__ __forceinline__ f16x8_t mx4_f16x8(uint32_t w, f16x2_t s2) {
  const E2m1Hi hb = e2m1_hi_bytes(w);
  const uint32_t ht = hb.ht, hu = hb.hu;
  const f16x2_t a = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0u, ht, kSelPairLo)) * s2;
  const f16x2_t b = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0u, hu, kSelPairLo)) * s2;
  const f16x2_t c = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0u, ht, kSelPairHi)) * s2;
  const f16x2_t d = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0u, hu, kSelPairHi)) * s2;
  f16x8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// MXFP4 on the MFMA path over every ue8m0 exponent.  The fp16 operand is
// e2m1 * 2^(e - 127 - shift), with shift chosen per weight row (over the
// groups a workgroup contracts, agreed by the two lanes feeding that output
// column) so that the row's largest finite exponent lands on kMxTopExp = 140,
// the top of the window 104..140 in which every e2m1 value times 2^(e - 127)
// is an exact fp16 number; the epilogue multiplies the fp32 accumulator by
// 2^shift (ldexp, exact unless the result leaves fp32's range).  A group
// within 36 of its row's largest exponent is therefore exact; one 37 below
// rounds once to fp16's subnormal grid; one 38 or more below contributes
// zero (its scale is no fp16 number: its weights are under 2^-22 * 2^shift,
// below 2^-34 of the row's largest weight).  e = 255 (NaN in the MX format)
// stays NaN, and a row of NaN groups only takes shift 0.
constexpr int kMxTopExp = 140;

// shift for a row whose largest finite exponent is emax (-1: none).
__device__ __forceinline__ int mx_row_shift(int emax) { return emax < 0 ? 0 : emax - kMxTopExp; }

// The fp16 scale 2^(e - 127 - shift), rounded to nearest even from the exact
// fp32 power of two (zero when e - shift <= 0; +inf past 142), NaN for e = 255.
__device__ __forceinline__ _Float16 e8m0_f16_shifted(uint32_t e, int shift) {
  const int eb = (int)e - shift;
  const float f = e == 255u ? __builtin_nanf("")
                            : eb <= 0 ? 0.0f : __uint_as_float((uint32_t)min(eb, 254) << 23);
  return (_Float16)f;
}

// int4 operands of one packed word for one-subtile MFMA tiles.  The word's
// bytes are reordered to (b0, b2, b1, b3), so its low nibbles read e0, e4, e2,
// e6 and its high nibbles e1, e5, e3, e7.  A byte 0000nnnn read as fp8 e4m3
// is n * 2^-9 exactly (n < 8 as a subnormal), so gfx950's packed fp8
// conversion at scale 2^9 turns each half of the masked word into an exact
// fp16 pair of nibbles in the operand order ([e0,e4], [e2,e6] / [e1,e5],
// [e3,e7]).  One fused multiply-add n * s + m8s with m8s = -8 s rounds
// (n - 8) * s once: the same operands as q4_f16x8 in fewer instructions,
// provided -8 s is itself an fp16 number, i.e. |s| <= 8188.  Beyond that
// m8s is -inf and every weight of the group with n >= 1 comes out -inf or
// NaN (q4_f16x8 still rounds each product once; for such scales weights of
// nibble 0 overflow on both).
__device__ __forceinline__ f16x8_t q4_f16x8_cvt(uint32_t w, f16x2_t s2, f16x2_t m8s2) {
  const uint32_t r = __builtin_amdgcn_perm(w, w, 0x03010200u);  // bytes b0, b2, b1, b3
  const uint32_t lo = r & 0x0F0F0F0Fu, hi = (r >> 4) & 0x0F0F0F0Fu;
  const f16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, false);  // [e0, e4]
  const f16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, true);   // [e2, e6]
  const f16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, false);  // [e1, e5]
  const f16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, true);   // [e3, e7]
  const f16x2_t ra = __builtin_elementwise_fma(a, s2, m8s2);
  const f16x2_t rb = __builtin_elementwise_fma(b, s2, m8s2);
  const f16x2_t rc = __builtin_elementwise_fma(c, s2, m8s2);
  const f16x2_t rd = __builtin_elementwise_fma(d, s2, m8s2);
  f16x8_t o;
  o[0] = ra[0]; o[1] = ra[1]; o[2] = rb[0]; o[3] = rb[1];
  o[4] = rc[0]; o[5] = rc[1]; o[6] = rd[0]; o[7] = rd[1];
  return o;
}

// The two e2m1 codes of byte B of w (low nibble first) as an fp16 pair, by
// gfx950's packed fp4 conversion with unit scale: every e2m1 value is an
// fp16 number, so the pair is exact.
template <int B>
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, B));
}

// MXFP4 operands of one packed word for one-subtile MFMA tiles, where the
// decode VALU outweighs the MFMA work of a K step: the packed fp4 conversion
// at unit scale gives the exact fp16 pairs [e0,e1], [e2,e3], [e4,e5], [e6,e7]
// (one per byte, low nibble first), one v_perm_b32 per pair regroups them
// into the operand order of mx4_f16x8, and the packed multiply by [s, s]
// rounds the exact product once: the same operands as mx4_f16x8, with fewer
// instructions.  (Beside the MFMA work of wider tiles the table decode of
// mx4_f16x8 measured faster.)
__device__ __forceinline__ f16x8_t mx4_f16x8_cvt(uint32_t w, f16x2_t s2) {
  constexpr uint32_t kLo = 0x05040100u, kHi = 0x07060302u;  // [src1, src0] low / high halves
  const uint32_t p01 = e2m1_pair<0>(w), p23 = e2m1_pair<1>(w);
  const uint32_t p45 = e2m1_pair<2>(w), p67 = e2m1_pair<3>(w);
  const f16x2_t a = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(p45, p01, kLo)) * s2;
  const f16x2_t b = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(p45, p01, kHi)) * s2;
  const f16x2_t c = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(p67, p23, kLo)) * s2;
  const f16x2_t d = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(p67, p23, kHi)) * s2;
  f16x8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// int4 decode, fp16 offset form (the down GEMV): 16-bit halves 0x64 0e = the
// exact fp16 value 1024 + e, in the pair order of q4_bf16_pairs.
__device__ __forceinline__ Q4Pairs q4_f16_pairs(uint32_t w) { return q4_pairs_with(w, 0x64646464u); }

__device__ __forceinline__ float half_bits_to_f32(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)v);
}

// ue8m0 group exponent e -> 2^(e - 127) in fp32 (the GEMV's MXFP4 scale):
// e << 23 for 1 <= e <= 254, 2^-127 (an fp32 subnormal) for e = 0, NaN for
// e = 255.  Exact for every e.
__device__ __forceinline__ float e8m0_f32(uint32_t e) {
  return __uint_as_float(e == 0 ? 0x00400000u : e == 255 ? 0x7FC00000u : e << 23);
}

// Position, within an aligned block of 8, at which element i is stored in the
// MFMA kernels' fp16 activation buffers (inverse of the order 0,4,1,5,2,6,3,7).
__device__ __forceinline__ int perm8_pos(int i) { return ((i & 3) << 1) | (i >> 2); }

// Eight bf16 activations (natural order, 16 bytes) -> eight fp16 in the MFMA
// operand order 0,4,1,5,2,6,3,7: dword d of the result holds elements d and
// d+4.  bf16 -> fp32 is exact; fp32 -> fp16 rounds to nearest even, which is
// exact for |x| in [2^-14, 65504] and within 2^-25 below.
__device__ __forceinline__ u32x4_t bf16x8_to_f16_perm8(u32x4_t v) {
  u32x4_t r;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t lo = (v[d >> 1] >> (16 * (d & 1))) & 0xFFFFu;         // element d
    const uint32_t hi = (v[(d + 4) >> 1] >> (16 * (d & 1))) & 0xFFFFu;   // element d + 4
    const f16x2_t h = {(_Float16)bf16_to_f32(lo), (_Float16)bf16_to_f32(hi)};
    r[d] = __builtin_bit_cast(uint32_t, h);
  }
  return r;
}

__device__ __forceinline__ float sigmoidf_acc(float z) { return 1.0f / (1.0f + expf(-z)); }

}  // namespace moe
