// Small helper kernels: the fp16 activation copy for the MFMA path and the
// int4 decode test hook.
#include "device.h"
#include "kernels.h"

namespace moe {

// x (bf16 [T][H]) -> fp16 [T][H] with every aligned block of 8 stored in the
// MFMA operand order (element i at position perm8_pos(i)).  bf16 -> fp16 is
// exact for |x| in [2^-14, 65504]; smaller magnitudes keep their value to
// within 2^-25 (fp16 subnormal spacing).  Also zeroes y (grid-stride).
__global__ __launch_bounds__(256) void convert_x16_kernel(const uint16_t* __restrict__ x,
                                                          int64_t blocks8,
                                                          uint16_t* __restrict__ x16,
                                                          float* __restrict__ y_zero,
                                                          int64_t y_elems) {
  const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t i = gid; i < blocks8; i += nthr) {
    const uint4 v = reinterpret_cast<const uint4*>(x)[i];
    const uint32_t nat[4] = {v.x, v.y, v.z, v.w};
    _Float16 out[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t b = (nat[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      out[perm8_pos(j)] = (_Float16)bf16_to_f32(b);
    }
    reinterpret_cast<uint4*>(x16)[i] = __builtin_bit_cast(uint4, out);
  }
  if (y_zero)
    for (int64_t i = gid; i < y_elems; i += nthr) y_zero[i] = 0.f;
}

hipError_t launch_convert_x16(const uint16_t* x, int T, int H, uint16_t* x16, float* y_zero,
                              int64_t y_elems, const Launch& L) {
  const int64_t blocks8 = (int64_t)T * H / 8;
  const int64_t work = blocks8 > y_elems ? blocks8 : y_elems;
  int grid = (int)((work + 255) / 256);
  if (grid > 8192) grid = 8192;
  if (grid < 1) grid = 1;
  MOE_LAUNCH(L, convert_x16_kernel, dim3(grid), dim3(256), 0, x, blocks8, x16, y_zero,
                     y_elems);
  return hipGetLastError();
}

// Decode one plane with the kernels' own routines.  One thread per packed
// 32-bit word (8 nibbles).
__global__ __launch_bounds__(256) void debug_dequant_kernel(const uint8_t* __restrict__ q,
                                                            const uint16_t* __restrict__ s,
                                                            int N, int K, int mode,
                                                            float* __restrict__ out) {
  const int64_t words = (int64_t)N * K / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= words) return;
  const int64_t n = i / (K / 8);
  const int kk0 = (int)(i % (K / 8)) * 8;
  const uint32_t wv = reinterpret_cast<const uint32_t*>(q)[i];
  const uint16_t sb = s[n * (K / 32) + kk0 / 32];
  float* o = out + n * K + kk0;
  if (mode == 0) {
    // bf16 offset form: pair j holds elements j and j+4 as 128 + nibble.
    const Q4Pairs p = q4_bf16_pairs(wv);
    const float sc = (float)__builtin_bit_cast(_Float16, sb);
    const uint32_t pr[4] = {p.p0, p.p1, p.p2, p.p3};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = bf16_to_f32(pr[j] & 0xFFFF), hi = bf16_to_f32(pr[j] >> 16);
      o[j] = (lo - 136.0f) * sc;
      o[j + 4] = (hi - 136.0f) * sc;
    }
  } else {
    const _Float16 sh = __builtin_bit_cast(_Float16, sb);
    const f16x2_t s2 = {sh, sh};
    const f16x8_t v = q4_f16x8(wv, s2);
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = (float)v[perm8_pos(j)];
  }
}

hipError_t launch_debug_dequant(const uint8_t* q, const uint16_t* s, int N, int K, int mode,
                                float* out, const Launch& L) {
  const int64_t words = (int64_t)N * K / 8;
  MOE_LAUNCH(L, debug_dequant_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0,
                     q, s, N, K, mode, out);
  return hipGetLastError();
}

}  // namespace moe
