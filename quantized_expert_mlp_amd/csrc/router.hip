// Router: logits GEMM (fp32 MFMA) and softmax -> top-k -> renormalise
// (one wave64 per token).
//
// Sources: the dasLLAMA vulkan PR #3988 routed-block commits (router GEMM over
// the normed rows and the f32 router plane, with a gated shared expert's gate
// row after the expert rows; per-row top-k, position-major picks and
// weights), and the vllm.cpp PR #481 warp router (one warp per token with the
// whole logit row in registers, a single read of the row, no shared memory,
// k rounds of arg-max then mask).
#include "device.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Logits L[t][e] = sum_h x[t][h] * Wr[e][h], plus column E = x[t] . g when a
// gate row is given.  One workgroup computes a 16-token x 16-row tile with
// v_mfma_f32_16x16x4_f32; its four waves split H in interleaved 16-wide
// chunks and their partial tiles are added through LDS.  Within a chunk lane
// (i, q) = (lane % 16, lane / 16) feeds A[i][q] = x[t0+i][c+4q+r] and
// B[q][i] = Wr[e0+i][c+4q+r] to the r-th of four MFMAs, so the four MFMAs
// together contract the 16 inputs c..c+15 (each lane reads 4 consecutive
// inputs with one vector load).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ wr,
                                                            const float* __restrict__ gate_row,
                                                            int T, int H, int E, float* out,
                                                            int ld) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, q = lane >> 4;
  const int t = blockIdx.x * 16 + i;
  const int e = blockIdx.y * 16 + i;
  const uint16_t* xrow = (t < T) ? x + (int64_t)t * H : nullptr;
  const float* wrow = nullptr;
  if (e < E) wrow = wr + (int64_t)e * H;
  else if (e == E && gate_row) wrow = gate_row;

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int c = wave * 16; c < H; c += 64) {
    const int kk = c + 4 * q;
    float a[4] = {0.f, 0.f, 0.f, 0.f}, b[4] = {0.f, 0.f, 0.f, 0.f};
    if (xrow) {
      const uint2 v = *reinterpret_cast<const uint2*>(xrow + kk);
      a[0] = __uint_as_float(v.x << 16);
      a[1] = __uint_as_float(v.x & 0xFFFF0000u);
      a[2] = __uint_as_float(v.y << 16);
      a[3] = __uint_as_float(v.y & 0xFFFF0000u);
    }
    if (wrow) {
      const float4 v = *reinterpret_cast<const float4*>(wrow + kk);
      b[0] = v.x; b[1] = v.y; b[2] = v.z; b[3] = v.w;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], b[r], acc, 0, 0, 0);
  }

  __shared__ f32x4_t part[4][64];
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4_t s = part[0][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) s += part[w][lane];
    // D[4*(lane/16) + r][lane % 16]: row = token, column = router row.
    const int col = blockIdx.y * 16 + i;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = blockIdx.x * 16 + 4 * q + r;
      if (row < T && col < ld) out[(int64_t)row * ld + col] = s[r];
    }
  }
}

hipError_t launch_router_logits(const uint16_t* x, const float* wr, const float* gate_row, int T,
                                int H, int E, float* out, int ld, hipStream_t st) {
  dim3 grid((T + 15) / 16, (ld + 15) / 16);
  hipLaunchKernelGGL(router_logits_kernel, grid, dim3(256), 0, st, x, wr, gate_row, T, H, E, out,
                     ld);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k.  Expert e lives in lane e % 64, register e / 64 (V registers, E <=
// 64 V).  Each of the k rounds takes the arg-max of what is left - larger
// logit first, lower expert index among equal logits - by a lane-local scan
// followed by a 6-step xor butterfly, which leaves the same winner in every
// lane because (value desc, index asc) is a total order; the owning lane
// then masks the winner.  Pick j stays in lane j.  Weights are
// exp(L_j - L_0) / sum_j' exp(L_j' - L_0) evaluated in fp64 (exact logit
// differences, one rounding to fp32 at the end).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return bi < 0 || (i >= 0 && (v > bv || (v == bv && i < bi)));
}

template <int V>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int ld,
                                                   int T, int E, int k, float route_scale,
                                                   int32_t* __restrict__ idx,
                                                   float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (int64_t)t * ld;
  float val[V];
  bool live[V];
#pragma unroll
  for (int r = 0; r < V; ++r) {
    const int e = lane + 64 * r;
    live[r] = e < E;
    val[r] = live[r] ? row[e] : 0.f;
  }
  float my_val = 0.f;
  int my_idx = -1;
  for (int j = 0; j < k; ++j) {
    float bv = 0.f;
    int bi = -1;
#pragma unroll
    for (int r = 0; r < V; ++r)
      if (live[r] && (bi < 0 || val[r] > bv)) {  // ascending index: strict > keeps ties low
        bv = val[r];
        bi = lane + 64 * r;
      }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi >= 0 && (bi & 63) == lane) live[bi >> 6] = false;
    if (lane == j) {
      my_val = bv;
      my_idx = bi;
    }
  }
  const double l0 = (double)__shfl(my_val, 0, 64);
  const double ex = (lane < k) ? exp((double)my_val - l0) : 0.0;
  double den = ex;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o, 64);
  if (lane < k) {
    idx[(int64_t)t * k + lane] = my_idx;
    w[(int64_t)t * k + lane] = (float)((double)route_scale * ex / den);
  }
}

hipError_t launch_topk(const float* logits, int ld, int T, int E, int k, float route_scale,
                       int32_t* idx, float* w, hipStream_t st) {
  dim3 grid((T + 3) / 4);
  const int V = (E + 63) / 64;
  switch (V) {
    case 1: hipLaunchKernelGGL(topk_kernel<1>, grid, dim3(256), 0, st, logits, ld, T, E, k, route_scale, idx, w); break;
    case 2: hipLaunchKernelGGL(topk_kernel<2>, grid, dim3(256), 0, st, logits, ld, T, E, k, route_scale, idx, w); break;
    case 3: hipLaunchKernelGGL(topk_kernel<3>, grid, dim3(256), 0, st, logits, ld, T, E, k, route_scale, idx, w); break;
    case 4: hipLaunchKernelGGL(topk_kernel<4>, grid, dim3(256), 0, st, logits, ld, T, E, k, route_scale, idx, w); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
