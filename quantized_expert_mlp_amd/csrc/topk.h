// Softmax -> top-k -> renormalise for one token on one wave64 (shared by the
// routing kernels and the small-batch routing prologue of the gate/up GEMV).
//
// Source: the vllm.cpp PR #481 warp router (one warp per token with the whole
// logit row in registers, a single read of the row, no shared memory, k
// rounds of arg-max then mask), re-shaped for wave64 and DPP.
#pragma once

#include "device.h"
#include "kernels.h"

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

// max(v, v of the DPP source lane); lanes outside ROW_MASK read INT_MIN
// (the identity) and keep v.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int imax_step(int v) {
  return max(v, __builtin_amdgcn_update_dpp((int)0x80000000, v, CTRL, ROW_MASK, 0xF, false));
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
__device__ void topk_group_variant(const float* __restrict__ logits, int ld, int T, int t0, int E,
                                   int k, const RouterSpec& rs, int32_t* __restrict__ idx,
                                   float* __restrict__ w, int32_t* idx_lds, float* w_lds,
                                   int lds_t0, int* lane_pick);

// need_w = false: the caller uses the picks only (w and w_lds are not
// written); with expert top-p on, the weights decide the picks and are
// formed anyway.  lane_pick, when non-null, receives in each lane the pick
// its group lane holds (group lane j < k: pick j, -1 if dropped; others -1).
// rounds < k (one token per wave, need_w false, no top-p, plain softmax
// router; ignored otherwise): stop after the first `rounds` picks, which
// are final (pick j is decided in round j); only the first `rounds` lanes
// are then written.
template <int V, int G>
__device__ __forceinline__ void topk_group(const float* __restrict__ logits, int ld, int T, int t0,
                                           int E, int k, const RouterSpec& rs,
                                           int32_t* __restrict__ idx, float* __restrict__ w,
                                           int32_t* idx_lds = nullptr, float* w_lds = nullptr,
                                           int lds_t0 = 0, bool need_w = true,
                                           int* lane_pick = nullptr, int rounds = 64) {
  static_assert(G == 16 || G == 32 || G == 64, "group size");
  if (rs.variant()) {  // uniform over the launch
    topk_group_variant<V, G>(logits, ld, T, t0, E, k, rs, idx, w, idx_lds, w_lds, lds_t0,
                             lane_pick);
    return;
  }
  const float route_scale = rs.route_scale, top_p = rs.top_p;
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
  if constexpr (G == 64) {
    // One token per wave: each round is a plain max over the wave, then the
    // winner is the lowest expert holding that value - registers in
    // ascending order, inside a register the lowest lane of the ballot -
    // found with scalar bit scans.  The max runs on integer keys that order
    // like the logits (sign-magnitude flipped to two's complement, -0 keyed
    // as +0 so that key equality is float equality), where each DPP step is
    // one integer max.
    int key[V];
#pragma unroll
    for (int r = 0; r < V; ++r) {
      const int bits = __float_as_int(val[r]);
      key[r] = bits == (int)0x80000000 ? 0 : bits < 0 ? bits ^ 0x7FFFFFFF : bits;
    }
    constexpr int kRetiredKey = (int)0x80000000;  // below -inf's key
    const int nr = (!need_w && !(top_p > 0.f && top_p < 1.f)) ? min(rounds, k) : k;
    for (int j = 0; j < nr; ++j) {
      int m = key[0];
#pragma unroll
      for (int r = 1; r < V; ++r) m = max(m, key[r]);
      m = imax_step<kDppXor1>(m);
      m = imax_step<kDppXor2>(m);
      m = imax_step<kDppHalfMirror>(m);
      m = imax_step<kDppMirror>(m);
      m = imax_step<kDppBcast15, 0xA>(m);
      m = imax_step<kDppBcast31, 0x8>(m);
      m = __builtin_amdgcn_readlane(m, 63);
      int wr = V, wl = 0;
#pragma unroll
      for (int r = V - 1; r >= 0; --r) {
        const uint64_t hit = __builtin_amdgcn_ballot_w64(key[r] == m);
        if (hit != 0) {
          wr = r;
          wl = (int)__builtin_ctzll(hit);
        }
      }
#pragma unroll
      for (int r = 0; r < V; ++r) {
        const bool mine = r == wr && lane == wl;
        key[r] = mine ? kRetiredKey : key[r];
        val[r] = mine ? ninf : val[r];
      }
      const float mv = __int_as_float(m < 0 ? m ^ 0x7FFFFFFF : m);
      my_val = lane == j ? mv : my_val;
      my_idx = lane == j ? wr * 64 + wl : my_idx;
    }
  } else {
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
  }
  if (!need_w && !(top_p > 0.f && top_p < 1.f)) {
    const int done = G == 64 ? min(rounds, k) : k;  // picks formed
    if (tok && gl < done) {
      if (idx) idx[(int64_t)t * k + gl] = my_idx;
      if (idx_lds) idx_lds[(t - lds_t0) * k + gl] = my_idx;
    }
    if (lane_pick) *lane_pick = tok && gl < done ? my_idx : -1;
    return;
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
  if (lane_pick) *lane_pick = tok && gl < k ? (keep ? my_idx : -1) : -1;
}

// Router variants (the dasLLAMA PR's MoE seat lists a non-softmax gate and a
// router or selection bias among the shapes it declines, without defining
// them; the vllm.cpp PR's dispatch names the grouped noaux_tc router; read
// as the published DeepSeek-V3 routing): score s_e = softmax(L)_e (rs.score
// 0) or sigmoid(L_e) (rs.score 1) in fp64, selection key s_e + b_e (b =
// rs.bias, zero when null); with rs.n_group > 1 the experts form n_group
// groups of E / n_group consecutive experts, a group scores the sum of its
// two largest keys, and only the experts of the rs.topk_group best groups
// (the lower group index winning a tie) stay in the selection; the k
// largest keys in rank order with the lower index winning a tie, and
// weights from the picks' unbiased scores renormalised, times route_scale:
//   w_j = route_scale * s_j / sum_j' s_j'.
// Same lane mapping as topk_group; the keys are fp64, so each round's
// arg-max is a xor butterfly of (key, index, score) over the group's lanes.
// Group scores: per expert group, each lane's two largest keys of that
// group, merged by a xor butterfly; group g's score then sits in group lane
// g (n_group <= kMaxGroups <= G), and the kept groups are found with the
// same arg-max rounds over those lanes.  Top-p does not apply.
__device__ __forceinline__ bool beats_d(double ov, int oi, double bv, int bi) {
  return (ov > bv) | ((ov == bv) & (oi < bi));
}

template <int V, int G>
__device__ void topk_group_variant(const float* __restrict__ logits, int ld, int T, int t0, int E,
                                   int k, const RouterSpec& rs, int32_t* __restrict__ idx,
                                   float* __restrict__ w, int32_t* idx_lds, float* w_lds,
                                   int lds_t0, int* lane_pick) {
  const int lane = threadIdx.x & 63;
  const int gl = lane % G;
  const int t = t0 + lane / G;
  const bool tok = t < T;
  const double ninf = -__builtin_huge_val();
  float lg[V];
  bool live[V];
#pragma unroll
  for (int r = 0; r < V; ++r) {
    const int e = gl + G * r;
    live[r] = tok && e < E;
    lg[r] = live[r] ? logits[(int64_t)t * ld + e] : 0.f;
  }
  double sc[V];
  if (rs.score == 1) {
#pragma unroll
    for (int r = 0; r < V; ++r) sc[r] = live[r] ? 1.0 / (1.0 + exp(-(double)lg[r])) : 0.0;
  } else {
    // softmax over the row: max (exact in fp32), then the fp64 sum of exp
    float m = -__builtin_huge_valf();
#pragma unroll
    for (int r = 0; r < V; ++r) m = live[r] ? fmaxf(m, lg[r]) : m;
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    double den = 0.0;
#pragma unroll
    for (int r = 0; r < V; ++r) {
      sc[r] = live[r] ? exp((double)lg[r] - (double)m) : 0.0;
      den += sc[r];
    }
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) den += __shfl_xor(den, o, 64);
    den = tok ? den : 1.0;
#pragma unroll
    for (int r = 0; r < V; ++r) sc[r] /= den;
  }
  double key[V];
  int id[V];
#pragma unroll
  for (int r = 0; r < V; ++r) {
    const int e = gl + G * r;
    key[r] = live[r] ? sc[r] + (rs.bias ? (double)rs.bias[e] : 0.0) : ninf;
    id[r] = live[r] ? e : kRetired;
  }
  if (rs.n_group > 1) {  // uniform over the launch
    const int ng = rs.n_group, gsz = E / ng;
    double my_gs = ninf;  // group gl's score, held in group lane gl
    for (int g = 0; g < ng; ++g) {
      double a1 = ninf, a2 = ninf;  // this lane's two largest keys of group g
#pragma unroll
      for (int r = 0; r < V; ++r) {
        const int e = gl + G * r;
        const double kk = (live[r] && e / gsz == g) ? key[r] : ninf;
        a2 = fmax(a2, fmin(a1, kk));
        a1 = fmax(a1, kk);
      }
#pragma unroll
      for (int o = G / 2; o > 0; o >>= 1) {  // top two of both lanes' top twos
        const double b1 = __shfl_xor(a1, o, 64), b2 = __shfl_xor(a2, o, 64);
        const double n2 = fmax(fmin(a1, b1), fmax(a2, b2));
        a1 = fmax(a1, b1);
        a2 = n2;
      }
      const double gsc = gsz >= 2 ? a1 + a2 : a1;
      my_gs = gl == g ? gsc : my_gs;
    }
    uint32_t kept = 0;
    double gv = gl < ng ? my_gs : ninf;
    int gi = gl < ng ? gl : kRetired;
    for (int j = 0; j < rs.topk_group; ++j) {
      double bv = gv;
      int bi = gi;
#pragma unroll
      for (int o = G / 2; o > 0; o >>= 1) {
        const double ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        const bool take = beats_d(ov, oi, bv, bi);
        bv = take ? ov : bv;
        bi = take ? oi : bi;
      }
      kept |= 1u << bi;  // every lane of the group holds the winner
      const bool mine = gi == bi;
      gv = mine ? ninf : gv;
      gi = mine ? kRetired : gi;
    }
#pragma unroll
    for (int r = 0; r < V; ++r) {  // experts of the other groups leave the selection
      const int e = gl + G * r;
      const bool out = live[r] && !((kept >> (e / gsz)) & 1u);
      key[r] = out ? ninf : key[r];
      id[r] = out ? kRetired : id[r];
    }
  }
  int my_idx = -1;
  double my_s = 0.0;
  for (int j = 0; j < k; ++j) {
    double bv = key[0], bs = sc[0];
    int bi = id[0];
#pragma unroll
    for (int r = 1; r < V; ++r) {
      const bool take = beats_d(key[r], id[r], bv, bi);
      bv = take ? key[r] : bv;
      bi = take ? id[r] : bi;
      bs = take ? sc[r] : bs;
    }
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) {
      const double ov = __shfl_xor(bv, o, 64), os = __shfl_xor(bs, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      const bool take = beats_d(ov, oi, bv, bi);
      bv = take ? ov : bv;
      bi = take ? oi : bi;
      bs = take ? os : bs;
    }
#pragma unroll
    for (int r = 0; r < V; ++r) {
      const bool mine = id[r] == bi;  // every lane of the group holds the winner
      key[r] = mine ? ninf : key[r];
      id[r] = mine ? kRetired : id[r];
    }
    my_idx = gl == j ? bi : my_idx;
    my_s = gl == j ? bs : my_s;
  }
  double den = gl < k ? my_s : 0.0;
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) den += __shfl_xor(den, o, 64);
  if (tok && gl < k) {
    const float wv = (float)((double)rs.route_scale * my_s / den);
    if (idx) idx[(int64_t)t * k + gl] = my_idx;
    if (w) w[(int64_t)t * k + gl] = wv;
    if (idx_lds) idx_lds[(t - lds_t0) * k + gl] = my_idx;
    if (w_lds) w_lds[(t - lds_t0) * k + gl] = wv;
  }
  if (lane_pick) *lane_pick = tok && gl < k ? my_idx : -1;
}

// Lanes per token: the smallest group that holds the row in 4 registers and
// the k picks in its lanes.
__host__ __device__ constexpr int topk_group_lanes(int E, int k) {
  return (E <= 64 && k <= 16) ? 16 : (E <= 128 && k <= 32) ? 32 : 64;
}

}  // namespace moe
