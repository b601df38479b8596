// Softmax -> top-k -> renormalise for one token on one wave64 (shared by the
// routing kernels and the small-batch routing prologue of the gate/up GEMV).
//
// Source: the vllm.cpp PR #481 warp router (one warp per token with the whole
// logit row in registers, a single read of the row, no shared memory, k
// rounds of arg-max then mask), re-shaped for wave64 and DPP.
#pragma once

#include "device.h"

namespace moe {

// ---------------------------------------------------------------------------
// Top-k for one token on one wave.  Expert e lives in lane e % 64, register
// e / 64 (V registers, E <= 64 V).  Each of the k rounds takes the arg-max of
// what is left - larger logit first, lower expert index among equal logits -
// by a lane-local scan, a DPP all-reduce inside each 16-lane row and a
// 4-way pick across the rows' results (read as uniform values); because
// (value desc, index asc) is a total order every lane agrees on the winner,
// whose owning lane then masks it.  Pick j stays in lane j.  Weights are
// exp(L_j - L_0) / sum_j' exp(L_j' - L_0) evaluated in fp64 (exact logit
// differences, one rounding to fp32 at the end).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return bi < 0 || (i >= 0 && (v > bv || (v == bv && i < bi)));
}

template <int CTRL>
__device__ __forceinline__ void argmax_step(float& bv, int& bi) {
  const float ov = dpp<CTRL>(bv);
  const int oi = dpp_i<CTRL>(bi);
  if (better(ov, oi, bv, bi)) {
    bv = ov;
    bi = oi;
  }
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Writes idx[j], w[j] for j < k when those are non-null (global), and the
// same into idx_lds[j], w_lds[j] when those are non-null (LDS).
template <int V>
__device__ __forceinline__ void topk_wave(const float* __restrict__ row, int E, int k,
                                          float route_scale, int32_t* __restrict__ idx,
                                          float* __restrict__ w, int32_t* idx_lds,
                                          float* w_lds = nullptr) {
  const int lane = threadIdx.x & 63;
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
    argmax_step<kDppXor1>(bv, bi);
    argmax_step<kDppXor2>(bv, bi);
    argmax_step<kDppHalfMirror>(bv, bi);
    argmax_step<kDppMirror>(bv, bi);
    float cv = readlane_f(bv, 0);
    int ci = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
    for (int rw = 1; rw < 4; ++rw) {
      const float ov = readlane_f(bv, 16 * rw);
      const int oi = __builtin_amdgcn_readlane(bi, 16 * rw);
      if (better(ov, oi, cv, ci)) {
        cv = ov;
        ci = oi;
      }
    }
    if (ci >= 0 && (ci & 63) == lane) {
#pragma unroll
      for (int r = 0; r < V; ++r)
        if (r == (ci >> 6)) live[r] = false;
    }
    if (lane == j) {
      my_val = cv;
      my_idx = ci;
    }
  }
  const double l0 = (double)readlane_f(my_val, 0);
  const double ex = (lane < k) ? exp((double)my_val - l0) : 0.0;
  double den = ex;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o, 64);
  if (lane < k) {
    const float wv = (float)((double)route_scale * ex / den);
    if (idx) idx[lane] = my_idx;
    if (w) w[lane] = wv;
    if (idx_lds) idx_lds[lane] = my_idx;
    if (w_lds) w_lds[lane] = wv;
  }
}

}  // namespace moe
