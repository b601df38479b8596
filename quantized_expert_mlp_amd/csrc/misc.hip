// Small helper kernels: the fp16 activation copy for the MFMA path, the
// tiled weight packing and the int4 decode test hook.
#include "device.h"
#include "kernels.h"

namespace moe {

// x (bf16 [T][H]) -> fp16 [T][H] with every aligned block of 8 stored in the
// MFMA operand order 0,4,1,5,2,6,3,7 (bf16x8_to_f16_perm8).  Grid-stride.
__global__ __launch_bounds__(256) void convert_x16_kernel(const uint16_t* __restrict__ x,
                                                          int64_t blocks8,
                                                          uint16_t* __restrict__ x16) {
  const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < blocks8; i += nthr)
    reinterpret_cast<u32x4_t*>(x16)[i] =
        bf16x8_to_f16_perm8(reinterpret_cast<const u32x4_t*>(x)[i]);
}

hipError_t launch_convert_x16(const uint16_t* x, int T, int H, uint16_t* x16, const Launch& L) {
  const int64_t blocks8 = (int64_t)T * H / 8;
  int grid = (int)((blocks8 + 255) / 256);
  if (grid > 8192) grid = 8192;
  if (grid < 1) grid = 1;
  MOE_LAUNCH(L, convert_x16_kernel, dim3(grid), dim3(256), 0, x, blocks8, x16);
  return hipGetLastError();
}

// The residual step after the layer (the dasLLAMA PR's combine folded into
// add+rms): the down pass has already added the FFN row into the fp32
// residual r; this writes the next layer's input n = bf16(r * g / rms(r)),
// rms(r) = sqrt(mean(r^2) + eps).  One workgroup per row: four float4 per
// thread per pass, the sum of squares in fp32 (wave DPP sums, then LDS across
// the 4 waves), one IEEE divide and square root per row, then a second pass
// over the row (L2-resident) for the products, rounded to nearest even.
// Every thread of the 256-thread workgroup calls row_inv_rms; part holds 4
// floats.
__device__ __forceinline__ float row_inv_rms(const float4* __restrict__ r4, int n4, int H,
                                             float eps, float* part) {
  float ss = 0.f;
  for (int i = threadIdx.x; i < n4; i += 256) {
    const float4 v = r4[i];
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = group_sum<64>(ss);
  if ((threadIdx.x & 63) == 63) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  return 1.0f / sqrtf(tot / (float)H + eps);
}

__device__ __forceinline__ uint2 norm4_bf16(float4 v, float4 w, float inv) {
  const uint32_t b0 = f32_to_bf16_rne(v.x * inv * w.x), b1 = f32_to_bf16_rne(v.y * inv * w.y);
  const uint32_t b2 = f32_to_bf16_rne(v.z * inv * w.z), b3 = f32_to_bf16_rne(v.w * inv * w.w);
  return make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
}

__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ r,
                                                      const float* __restrict__ g, int H,
                                                      float eps, uint16_t* __restrict__ out) {
  __shared__ float part[4];
  const int64_t row = blockIdx.x;
  const float4* r4 = reinterpret_cast<const float4*>(r + row * H);
  const float4* g4 = reinterpret_cast<const float4*>(g);
  const int n4 = H / 4;
  const float inv = row_inv_rms(r4, n4, H, eps, part);
  uint2* o4 = reinterpret_cast<uint2*>(out + row * H);
  for (int i = threadIdx.x; i < n4; i += 256) o4[i] = norm4_bf16(r4[i], g4[i], inv);
}

hipError_t launch_rmsnorm(const float* r, const float* g, int T, int H, float eps, uint16_t* out,
                          const Launch& L) {
  MOE_LAUNCH(L, rmsnorm_kernel, dim3(T), dim3(256), 0, r, g, H, eps, out);
  return hipGetLastError();
}

// The same step with the next layer's router folded into its epilogue (the
// vllm.cpp PR's closing hypothesis: the router folded into the preceding
// kernel, fewer launches per step).  Workgroup (bx, by) takes token rows
// by*kFoldRouterRows .. +kFoldRouterRows-1: it normalises them exactly as
// rmsnorm_kernel does (every workgroup of a row block recomputes the norm
// from the L2-resident residual rows), keeps the bf16 rows in LDS, writes
// them to out when bx == 0, and wave w computes router row e = 4*bx + w of
// the next layer's logits, L[t][e] = sum_h float(n[t][h]) * wr[e][h] in fp32
// (16-byte router loads, a DPP sum across the wave).  Dynamic LDS:
// kFoldRouterRows * H bf16.
__global__ __launch_bounds__(256) void rmsnorm_router_kernel(
    const float* __restrict__ r, const float* __restrict__ g, int T, int H, float eps,
    uint16_t* __restrict__ out, const float* __restrict__ wr, int E, float* __restrict__ logits) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  __shared__ float part[kFoldRouterRows][4];
  const int t0 = blockIdx.y * kFoldRouterRows;
  const int nt = min(kFoldRouterRows, T - t0);
  const int n4 = H / 4;
  const float4* g4 = reinterpret_cast<const float4*>(g);
  for (int tt = 0; tt < nt; ++tt) {
    const float4* r4 = reinterpret_cast<const float4*>(r + (int64_t)(t0 + tt) * H);
    const float inv = row_inv_rms(r4, n4, H, eps, part[tt]);
    uint2* x4 = reinterpret_cast<uint2*>(xs + tt * H);
    uint2* o4 = reinterpret_cast<uint2*>(out + (int64_t)(t0 + tt) * H);
    for (int i = threadIdx.x; i < n4; i += 256) {
      const uint2 b = norm4_bf16(r4[i], g4[i], inv);
      x4[i] = b;
      if (blockIdx.x == 0) o4[i] = b;
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const float4* w4 = reinterpret_cast<const float4*>(wr + (int64_t)e * H);
  float acc[kFoldRouterRows];
#pragma unroll
  for (int tt = 0; tt < kFoldRouterRows; ++tt) acc[tt] = 0.f;
#pragma unroll 4
  for (int i = lane; i < n4; i += 64) {
    const float4 w = w4[i];
#pragma unroll
    for (int tt = 0; tt < kFoldRouterRows; ++tt) {
      if (tt < nt) {
        const uint2 b = reinterpret_cast<const uint2*>(xs + tt * H)[i];
        acc[tt] += bf16_to_f32(b.x & 0xFFFFu) * w.x + bf16_to_f32(b.x >> 16) * w.y +
                   bf16_to_f32(b.y & 0xFFFFu) * w.z + bf16_to_f32(b.y >> 16) * w.w;
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < kFoldRouterRows; ++tt) {
    const float v = group_sum<64>(acc[tt]);
    if (lane == 63 && tt < nt) logits[(int64_t)(t0 + tt) * E + e] = v;
  }
}

hipError_t launch_rmsnorm_router(const float* r, const float* g, int T, int H, float eps,
                                 uint16_t* out, const float* wr, int E, float* logits,
                                 const Launch& L) {
  if (!fold_router_served(T, H)) {
    // large batches: the norm launch, then the router-logits kernel over the
    // normed rows (the same logits, two launches)
    const Launch first{L.st, L.start, nullptr}, last{L.st, nullptr, L.stop};
    MOE_LAUNCH(first, rmsnorm_kernel, dim3(T), dim3(256), 0, r, g, H, eps, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_router_logits(out, wr, nullptr, T, H, E, logits, E, nullptr, last);
  }
  const dim3 grid((E + 3) / 4, (T + kFoldRouterRows - 1) / kFoldRouterRows);
  MOE_LAUNCH(L, rmsnorm_router_kernel, grid, dim3(256),
             (size_t)kFoldRouterRows * H * sizeof(uint16_t), r, g, T, H, eps, out, wr, E, logits);
  return hipGetLastError();
}

// Row layout -> tiled layout (see the moe_pack_weights contract): thread c
// moves destination q chunk c (16 bytes) and destination scale c (an fp16 or
// a ue8m0 byte, SE); per expert both number N*K/32.
template <typename SE>
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint8_t* __restrict__ sq,
                                                           const SE* __restrict__ ss,
                                                           int64_t total, int N, int K,
                                                           uint8_t* __restrict__ dq,
                                                           SE* __restrict__ ds) {
  const int64_t per = (int64_t)N * K / 32;
  const int nc = K / 64;
  const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += nthr) {
    const int64_t e = c / per, r = c % per;
    const int64_t tile = r / 64;
    const int within = (int)(r % 64), h = within / 32, j = within % 32;
    const int64_t b = tile / nc, cc = tile % nc;
    const int64_t row = e * N + 32 * b + j;
    reinterpret_cast<u32x4_t*>(dq)[c] =
        *reinterpret_cast<const u32x4_t*>(sq + row * (K / 2) + 32 * cc + 16 * h);
    ds[c] = ss[row * (K / 32) + 2 * cc + h];
  }
}

hipError_t launch_pack_weights(const uint8_t* sq, const void* ss, int E, int N, int K,
                               uint8_t* dq, void* ds, int fmt, const Launch& L) {
  const int64_t total = (int64_t)E * N * K / 32;
  int64_t grid = (total + 255) / 256;
  if (grid > 16384) grid = 16384;
  if (fmt == kFmtMxfp4)
    MOE_LAUNCH(L, pack_weights_kernel<uint8_t>, dim3((unsigned)grid), dim3(256), 0, sq,
               static_cast<const uint8_t*>(ss), total, N, K, dq, static_cast<uint8_t*>(ds));
  else
    MOE_LAUNCH(L, pack_weights_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, sq,
               static_cast<const uint16_t*>(ss), total, N, K, dq, static_cast<uint16_t*>(ds));
  return hipGetLastError();
}

// Streaming-read probe (the practical HBM read ceiling the GEMVs are held
// against): each thread reads 16-byte words of src with the nontemporal hint
// the GEMV weight stream uses, in a grid-stride loop, and folds them with
// xor.  The fold is stored only when it equals ~0 in every word, which keeps
// the loads alive without a store per thread.
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4_t* __restrict__ src,
                                                         int64_t words,
                                                         uint32_t* __restrict__ sink) {
  const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * nthr < words; i += 4 * nthr) {
    const u32x4_t a = __builtin_nontemporal_load(src + i);
    const u32x4_t b = __builtin_nontemporal_load(src + i + nthr);
    const u32x4_t c = __builtin_nontemporal_load(src + i + 2 * nthr);
    const u32x4_t d = __builtin_nontemporal_load(src + i + 3 * nthr);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < words; i += nthr) acc ^= __builtin_nontemporal_load(src + i);
  if ((acc[0] & acc[1] & acc[2] & acc[3]) == 0xFFFFFFFFu) sink[threadIdx.x] = acc[0];
}

hipError_t launch_read_probe(const void* src, int64_t bytes, int workgroups, uint32_t* sink,
                             const Launch& L) {
  MOE_LAUNCH(L, read_probe_kernel, dim3(workgroups), dim3(256), 0,
             static_cast<const u32x4_t*>(src), bytes / 16, sink);
  return hipGetLastError();
}

// Decode one plane with the kernels' own routines (the ones their main loops
// call), one thread per packed 32-bit word (8 nibbles), and write what each
// decoder stands for as fp32: the GEMV decoders' exact weight (their offset
// form and group scale undone exactly in fp32), the MFMA decoders' fp16
// operand widened.  The decoders' output orders are undone here: pairs
// (j, j+4) for the offset forms, natural pairs for e2m1_pair, the order
// 0,4,1,5,2,6,3,7 for the MFMA operands.
__global__ __launch_bounds__(256) void debug_dequant_kernel(const uint8_t* __restrict__ q,
                                                            const void* __restrict__ s,
                                                            int N, int K, int mode,
                                                            float* __restrict__ out) {
  const int64_t words = (int64_t)N * K / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= words) return;
  const int64_t n = i / (K / 8);
  const int kk0 = (int)(i % (K / 8)) * 8;
  const uint32_t wv = reinterpret_cast<const uint32_t*>(q)[i];
  const int64_t g = n * (K / 32) + kk0 / 32;
  float* o = out + n * K + kk0;
  if (mode >= kDebugMx4Gemv) {  // MXFP4: ue8m0 scale bytes
    const uint32_t e = static_cast<const uint8_t*>(s)[g];
    if (mode == kDebugMx4Gemv) {
      const float sc = e8m0_f32(e);
      const uint32_t pr[4] = {e2m1_pair<0>(wv), e2m1_pair<1>(wv), e2m1_pair<2>(wv),
                              e2m1_pair<3>(wv)};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[2 * j] = half_bits_to_f32(pr[j] & 0xFFFFu) * sc;
        o[2 * j + 1] = half_bits_to_f32(pr[j] >> 16) * sc;
      }
      return;
    }
    // the row's shift over all its groups, as a workgroup contracting the
    // whole row forms it; the operand widened and scaled back by 2^shift
    const uint8_t* srow = static_cast<const uint8_t*>(s) + n * (K / 32);
    int m = -1;
    for (int gg = 0; gg < K / 32; ++gg) m = (srow[gg] != 255 && srow[gg] > m) ? srow[gg] : m;
    const int shift = mx_row_shift(m);
    const _Float16 sh = e8m0_f16_shifted(e, shift);
    const f16x2_t s2 = {sh, sh};
    const f16x8_t v = mode == kDebugMx4Mfma ? mx4_f16x8(wv, s2) : mx4_f16x8_cvt(wv, s2);
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = ldexpf((float)v[perm8_pos(j)], shift);
    return;
  }
  const uint16_t sb = static_cast<const uint16_t*>(s)[g];
  if (mode == kDebugQ4GemvGateUp || mode == kDebugQ4GemvDown) {
    // offset forms: pair j holds elements j and j+4 as 128 + e (bf16) or
    // 1024 + e (fp16)
    const bool gu = mode == kDebugQ4GemvGateUp;
    const Q4Pairs p = gu ? q4_bf16_pairs(wv) : q4_f16_pairs(wv);
    const float sc = half_bits_to_f32(sb), off = gu ? 136.0f : 1032.0f;
    const uint32_t pr[4] = {p.p0, p.p1, p.p2, p.p3};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = pr[j] & 0xFFFFu, hi = pr[j] >> 16;
      o[j] = ((gu ? bf16_to_f32(lo) : half_bits_to_f32(lo)) - off) * sc;
      o[j + 4] = ((gu ? bf16_to_f32(hi) : half_bits_to_f32(hi)) - off) * sc;
    }
    return;
  }
  const _Float16 sh = __builtin_bit_cast(_Float16, sb);
  const f16x2_t s2 = {sh, sh};
  // the one-subtile tiles' -8 s, formed as the GEMM forms it
  const f16x2_t m8s2 = s2 * f16x2_t{(_Float16)-8.0f, (_Float16)-8.0f};
  const f16x8_t v = mode == kDebugQ4Mfma ? q4_f16x8(wv, s2) : q4_f16x8_cvt(wv, s2, m8s2);
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = (float)v[perm8_pos(j)];
}

hipError_t launch_debug_dequant(const uint8_t* q, const void* s, int N, int K, int mode,
                                float* out, const Launch& L) {
  const int64_t words = (int64_t)N * K / 8;
  MOE_LAUNCH(L, debug_dequant_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0,
                     q, s, N, K, mode, out);
  return hipGetLastError();
}

}  // namespace moe
