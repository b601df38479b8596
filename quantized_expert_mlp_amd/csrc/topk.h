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
// Top-k for 64/G tokens on one wave: token g of the wave owns the aligned
// group of G lanes g*G .. g*G+G-1 (G = 16, 32 or 64); its expert e lives in
// group lane e % G, register e / G (V registers, E <= G*V; k <= G).  Each of
// the k rounds takes the arg-max of what is left - larger logit first, lower
// expert index among equal logits - by a lane-local scan, a DPP all-reduce
// inside each 16-lane row and, for G > 16, DPP row broadcasts that fold the
// rows into the group's last lane, read back as a uniform value.  All
// selects are branch-free.  Because (value desc, index asc) is a total order
// every lane of a group agrees on the winner, whose owning lane retires it
// (value -inf, index past every expert).  Pick j stays in group lane j.
// Weights are exp(L_j - L_0) / sum_j' exp(L_j' - L_0) evaluated in fp64
// (exact logit differences, one rounding to fp32 at the end).  Logits must be
// finite (an out-of-range lane and a retired pick read as -inf).
// ---------------------------------------------------------------------------
constexpr int kRetired = 0x7FFFFFFF;

// (ov, oi) beats (bv, bi): larger value, or equal value and lower index.
__device__ __forceinline__ bool beats(float ov, int oi, float bv, int bi) {
  return (ov > bv) | ((ov == bv) & (oi < bi));
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ void argmax_step(float& bv, int& bi) {
  // lanes outside ROW_MASK keep their own pair (update_dpp's old value)
  const float ov = __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(bv), __float_as_int(bv), CTRL, ROW_MASK, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(bi, bi, CTRL, ROW_MASK, 0xF, false);
  const bool take = beats(ov, oi, bv, bi);
  bv = take ? ov : bv;
  bi = take ? oi : bi;
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Tokens t0 .. t0 + 64/G - 1 (those below T) of a logits matrix with row
// stride ld.  Writes idx[t*k + j], w[t*k + j] for j < k when those are
// non-null (global), and the same into idx_lds / w_lds (indexed t*k + j, t
// relative to lds_t0) when those are non-null (LDS).
//
// Expert top-p (0 < top_p < 1; other values keep all k): pick j stays while
// the full-softmax probability of the picks ranked above it is below top_p;
// the others are written as index -1, weight 0, and the weights renormalise
// over the kept picks.  The full softmax mass is the picks' terms plus the
// logits still in the registers (selection retires picks to -inf), in fp64.
template <int V, int G>
__device__ __forceinline__ void topk_group(const float* __restrict__ logits, int ld, int T, int t0,
                                           int E, int k, float route_scale, float top_p,
                                           int32_t* __restrict__ idx, float* __restrict__ w,
                                           int32_t* idx_lds = nullptr, float* w_lds = nullptr,
                                           int lds_t0 = 0) {
  static_assert(G == 16 || G == 32 || G == 64, "group size");
  const int lane = threadIdx.x & 63;
  const int g = lane / G, gl = lane % G;
  const int t = t0 + g;
  const bool tok = t < T;
  const float ninf = -__builtin_huge_valf();
  float val[V];
  int id[V];
#pragma unroll
  for (int r = 0; r < V; ++r) {
    const int e = gl + G * r;
    const bool live = tok && e < E;
    val[r] = live ? logits[(int64_t)t * ld + e] : ninf;
    id[r] = live ? e : kRetired;
  }
  float my_val = 0.f;
  int my_idx = -1;
  for (int j = 0; j < k; ++j) {
    float bv = val[0];
    int bi = id[0];
#pragma unroll
    for (int r = 1; r < V; ++r) {
      const bool take = beats(val[r], id[r], bv, bi);
      bv = take ? val[r] : bv;
      bi = take ? id[r] : bi;
    }
    argmax_step<kDppXor1>(bv, bi);
    argmax_step<kDppXor2>(bv, bi);
    argmax_step<kDppHalfMirror>(bv, bi);
    argmax_step<kDppMirror>(bv, bi);        // every lane of a row: the row's winner
    if (G >= 32) argmax_step<kDppBcast15, 0xA>(bv, bi);  // rows 1, 3 also see rows 0, 2
    if (G == 64) argmax_step<kDppBcast31, 0x8>(bv, bi);  // row 3 also sees rows 0-1
    // the group's winner sits in its last lane; bring it to every lane
    float cv = bv;
    int ci = bi;
    if (G == 64) {
      cv = readlane_f(bv, 63);
      ci = __builtin_amdgcn_readlane(bi, 63);
    } else if (G == 32) {
      const float c0 = readlane_f(bv, 31), c1 = readlane_f(bv, 63);
      const int i0 = __builtin_amdgcn_readlane(bi, 31), i1 = __builtin_amdgcn_readlane(bi, 63);
      cv = g ? c1 : c0;
      ci = g ? i1 : i0;
    }
#pragma unroll
    for (int r = 0; r < V; ++r) {
      const bool mine = id[r] == ci;  // the winner's own register (ids are distinct)
      val[r] = mine ? ninf : val[r];
      id[r] = mine ? kRetired : id[r];
    }
    my_val = gl == j ? cv : my_val;
    my_idx = gl == j ? ci : my_idx;
  }
  // weights: group lane 0 holds the top logit
  const double l0 = (double)__shfl(my_val, g * G, 64);
  double ex = (gl < k) ? exp((double)my_val - l0) : 0.0;
  bool keep = gl < k;
  if (top_p > 0.f && top_p < 1.f) {
    double all = ex;
#pragma unroll
    for (int r = 0; r < V; ++r) all += exp((double)val[r] - l0);  // retired: exp(-inf) = 0
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) all += __shfl_xor(all, o, 64);
    // inclusive prefix of the picks' terms over the group's lanes
    double cum = ex;
#pragma unroll
    for (int o = 1; o < G; o <<= 1) {
      const double v = __shfl_up(cum, o, G);
      cum += gl >= o ? v : 0.0;
    }
    double above = __shfl_up(cum, 1, G);
    above = gl == 0 ? 0.0 : above;
    keep = keep && above / all < (double)top_p;
    ex = keep ? ex : 0.0;
  }
  double den = ex;
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) den += __shfl_xor(den, o, 64);
  if (tok && gl < k) {
    const float wv = keep ? (float)((double)route_scale * ex / den) : 0.0f;
    const int32_t iv = keep ? my_idx : -1;
    if (idx) idx[(int64_t)t * k + gl] = iv;
    if (w) w[(int64_t)t * k + gl] = wv;
    if (idx_lds) idx_lds[(t - lds_t0) * k + gl] = iv;
    if (w_lds) w_lds[(t - lds_t0) * k + gl] = wv;
  }
}

// Lanes per token: the smallest group that holds the row in 4 registers and
// the k picks in its lanes.
__host__ __device__ constexpr int topk_group_lanes(int E, int k) {
  return (E <= 64 && k <= 16) ? 16 : (E <= 128 && k <= 32) ? 32 : 64;
}

}  // namespace moe
