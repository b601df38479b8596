// CPU oracle for the fused int4 / MXFP4 Mixture-of-Experts layer.
//
// TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
// call this file: only the tests, the package's smoke check and the
// benchmark's CPU-baseline leg use it.  It shares no source with the HIP
// library: no headers, helpers or tables in common.
//
// It is the plain definition of what the layer computes, written as slow,
// obviously correct loops with fp64 accumulation, outputs rounded to fp32 at
// the end.  Sources (the web pages this layer is built from):
//   [colibri]  colibri PR #418, "Vulkan backend: expert tier + dense + MLA
//              attention on any Vulkan 1.2 GPU": the Correctness section
//              (int4 offset-binary nibble-8, CPU byte layout) and the later
//              grouped-scale revision (one scale per gs inputs, fmt=4).
//   [dasllama] daScript PR #3988, "dasLLAMA vulkan: a MoE that fits the card
//              serves on the whole-model resident driver": the commit notes on
//              the routed block (router GEMM, per-row top-k renormalised and
//              scaled, bucket schedule in slot order, combine), on the shared
//              expert (one region over every row, sigmoid gate logit as one
//              more router row) and on the combine folded into add+rms (the
//              FFN row summed as gated shared row first, then the slots in
//              order).
//   [dasllama-fold] the same dasLLAMA PR's commit folding the combine into the
//              residual step: the add+rms after the routed block adds the FFN
//              row (gated shared row, then the slots in order) to the
//              residual and norms the row for the next layer.
//   [vllmcpp]  vllm.cpp PR #481, "gate(#378): the first DEVICE run of the
//              warp MoE router": the ungated softmax router with top-k, k
//              passes of mask-and-reseed over the logit row.
//   [colibri-mx] the same colibri PR, the later comment adding fmt=7: MXFP4
//              expert weights, an e2m1 nibble per weight and one ue8m0
//              exponent per 32-input group.  The two element formats are
//              those of the OCP Microscaling (MX) v1.0 specification, which
//              the pages name but do not define: e2m1 = 1 sign, 2 exponent
//              (bias 1), 1 mantissa bit, no inf/NaN; ue8m0 = an unsigned
//              8-bit biased exponent, 2^(e - 127), 0xFF = NaN.
// Where the pages leave a step open, the reading taken is stated at the
// function.
//
// Parity status: every function here is pinned by the CPU tests
// (tests/test_oracle_*.py) against brute force, closed forms and invariants.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

// IEEE-754 binary16 -> double, from the format's definition (1 sign bit, 5
// exponent bits with bias 15, 10 fraction bits; exponent 0 = subnormal).
double half_to_double(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int ex = (h >> 10) & 0x1f;
  const int frac = h & 0x3ff;
  double v;
  if (ex == 0)
    v = std::ldexp((double)frac, -24);  // 0.frac * 2^-14
  else if (ex == 31)
    v = frac ? NAN : INFINITY;
  else
    v = std::ldexp(1024.0 + frac, ex - 25);  // 1.frac * 2^(ex-15)
  return sign ? -v : v;
}

// bf16 is the top half of an IEEE binary32.
double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// Offset-binary int4 with grouped scales ([colibri] Correctness: each nibble
// stands for nibble minus eight, stored in the host's byte layout; grouped-scale
// revision: one scale covers gs consecutive inputs, gs a multiple of 8).
// Reading of the byte layout: element kk of a row sits in byte kk/2, the low
// nibble holding the even element.  Scales run along the input (K) axis,
// gs = 32.
inline double weight_int4(const uint8_t* q, const uint16_t* s, int64_t K, int64_t n, int64_t kk) {
  const uint8_t byte = q[n * (K / 2) + kk / 2];
  const int nib = (kk & 1) ? (byte >> 4) : (byte & 0xf);
  return (double)(nib - 8) * half_to_double(s[n * (K / 32) + kk / 32]);
}

// e2m1 from its bit fields: bit 3 sign, bits 2..1 exponent (bias 1), bit 0
// mantissa.  Exponent field 0 is subnormal: 0.m * 2^0 = m/2; otherwise
// 1.m * 2^(E-1).  All 16 codes are finite.
double e2m1_to_double(int nib) {
  const int sign = (nib >> 3) & 1;
  const int ex = (nib >> 1) & 3;
  const int man = nib & 1;
  const double v = (ex == 0) ? 0.5 * man : std::ldexp(1.0 + 0.5 * man, ex - 1);
  return sign ? -v : v;
}

// ue8m0: the byte is a biased exponent, value 2^(e - 127); 0xFF is NaN.
double e8m0_to_double(uint8_t e) { return e == 0xFF ? NAN : std::ldexp(1.0, (int)e - 127); }

// MXFP4 ([colibri-mx]): same byte layout as the int4 planes (element kk in
// byte kk/2, low nibble = even kk); element value e2m1(nibble) times the
// group's 2^(e - 127), one ue8m0 byte per 32 consecutive inputs, scales
// row-major [N][K/32] like the int4 fp16 scales.
inline double weight_mxfp4(const uint8_t* q, const uint8_t* s, int64_t K, int64_t n, int64_t kk) {
  const uint8_t byte = q[n * (K / 2) + kk / 2];
  const int nib = (kk & 1) ? (byte >> 4) : (byte & 0xf);
  return e2m1_to_double(nib) * e8m0_to_double(s[n * (K / 32) + kk / 32]);
}

// Weight formats: 0 = int4 with fp16 scales, 1 = MXFP4 with ue8m0 scales.
// s points at the scale plane in its own element type.
inline double weight(int fmt, const uint8_t* q, const void* s, int64_t K, int64_t n, int64_t kk) {
  return fmt == 1 ? weight_mxfp4(q, static_cast<const uint8_t*>(s), K, n, kk)
                  : weight_int4(q, static_cast<const uint16_t*>(s), K, n, kk);
}

// Bytes of one scale element.
inline int64_t scale_bytes(int fmt) { return fmt == 1 ? 1 : 2; }
inline const void* scale_at(int fmt, const void* s, int64_t elems) {
  return static_cast<const char*>(s) + elems * scale_bytes(fmt);
}

double sigmoid(double z) { return 1.0 / (1.0 + std::exp(-z)); }

// fp64 -> bf16 bits, rounded once to nearest with ties to even.  bf16 keeps 8
// significant bits and fp32's exponent range: normal values are rounded to 8
// significant bits, values below 2^-126 to a multiple of 2^-133 (subnormal
// spacing); magnitudes past the largest bf16 after rounding are +-inf.
uint16_t double_to_bf16(double v) {
  if (std::isnan(v)) return 0x7FC0;
  const double a = std::fabs(v);
  double r;
  if (a == 0.0 || std::isinf(a)) {
    r = a;
  } else {
    int e;
    std::frexp(a, &e);                      // a = m * 2^e, 0.5 <= m < 1
    const int q = std::max(e - 8, -133);    // weight of the last kept bit
    r = std::ldexp(std::nearbyint(std::ldexp(a, -q)), q);
  }
  const double kMax = std::ldexp(255.0, 120);  // (2 - 2^-7) * 2^127
  float f = r > kMax ? INFINITY : (float)r;    // r has <= 8 significant bits: exact
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)((u >> 16) | (std::signbit(v) ? 0x8000u : 0u));
}

// One expert's SwiGLU MLP in fp64: g = Wg.x, u = Wu.x, h = silu(g)*u,
// o = Wd.h ([colibri] Summary: the fused expert computes gate and up, the SiLU
// product, then down; silu(z) = z*sigmoid(z) applied to the gate row).
void expert_forward(int fmt, const uint8_t* qg, const void* sg, const uint8_t* qu,
                    const void* su, const uint8_t* qd, const void* sd,
                    int64_t H, int64_t I, const double* x, double* h, double* o) {
  for (int64_t n = 0; n < I; ++n) {
    double g = 0.0, u = 0.0;
    for (int64_t kk = 0; kk < H; ++kk) {
      g += weight(fmt, qg, sg, H, n, kk) * x[kk];
      u += weight(fmt, qu, su, H, n, kk) * x[kk];
    }
    h[n] = g * sigmoid(g) * u;
  }
  for (int64_t n = 0; n < H; ++n) {
    double acc = 0.0;
    for (int64_t kk = 0; kk < I; ++kk) acc += weight(fmt, qd, sd, I, n, kk) * h[kk];
    o[n] = acc;
  }
}

// Selection for one row of logits: experts ranked by logit, descending, the
// lower expert index winning a tie; the first k in rank order.  This is the
// k-pass mask-and-reseed selection of [vllmcpp] (each pass takes the arg-max
// of what is left).  Reading: the rank key is the logit itself (softmax is
// monotone, so ranking probabilities gives the same order up to rounding
// ties); IEEE comparison, so -0.0 and +0.0 tie.
void select_row(const float* L, int64_t E, int64_t k, int32_t* idx) {
  std::vector<char> taken(E, 0);
  for (int64_t j = 0; j < k; ++j) {
    int64_t best = -1;
    for (int64_t e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || L[e] > L[best]) best = e;  // strict: the lower index keeps a tie
    }
    taken[best] = 1;
    idx[j] = (int32_t)best;
  }
}

// Renormalised softmax weights over the selection: softmax over all E
// experts, restricted to the picks and renormalised to sum to one, times the
// routed scale ([dasllama] routed-block commit: the per-row top-k is checked
// against the CPU selection renormalised and then scaled; [vllmcpp]: the
// softmax router without expert groups).  The full
// softmax's denominator cancels in the renormalisation, so this is
//   w_j = scale * exp(L_j - L_0) / sum_{j'<k} exp(L_j' - L_0),
// with L_0 the top logit.  Computed in fp64.
void weights_row(const float* L, const int32_t* idx, int64_t k, double scale, double* w) {
  const double l0 = (double)L[idx[0]];
  double den = 0.0;
  for (int64_t j = 0; j < k; ++j) den += std::exp((double)L[idx[j]] - l0);
  for (int64_t j = 0; j < k; ++j) w[j] = scale * std::exp((double)L[idx[j]] - l0) / den;
}

// Expert top-p ([colibri] Measured performance: its end-to-end decode runs
// with "expert-routing top-p 0.7"; the page names the setting but does not
// define it).  Reading: after the top-k selection, the picks are taken in
// rank order while the full-softmax probability of the picks ranked above
// them is still below p (the first pick is always kept); the rest are dropped
// (index -1, weight 0) and the weights are renormalised over the kept picks,
// times the routed scale.  p outside (0, 1) keeps all k.  Probabilities are
// exp(L_j - L_0) / sum_e exp(L_e - L_0) over all E experts, in fp64.
// Returns the number of kept picks.
int64_t top_p_row(const float* L, int64_t E, int64_t k, double top_p, double scale, int32_t* idx,
                  double* w) {
  if (!(top_p > 0.0 && top_p < 1.0)) return k;
  const double l0 = (double)L[idx[0]];
  double all = 0.0;
  for (int64_t e = 0; e < E; ++e) all += std::exp((double)L[e] - l0);
  double above = 0.0, kept_den = 0.0;
  int64_t kept = 0;
  for (int64_t j = 0; j < k; ++j) {
    if (!(above / all < top_p)) break;
    const double ex = std::exp((double)L[idx[j]] - l0);
    above += ex;
    kept_den += ex;
    ++kept;
  }
  for (int64_t j = 0; j < k; ++j) {
    if (j < kept) {
      w[j] = scale * std::exp((double)L[idx[j]] - l0) / kept_den;
    } else {
      idx[j] = -1;
      w[j] = 0.0;
    }
  }
  return kept;
}

// Router variants that [dasllama]'s MoE seat lists as declined shapes (a
// non-softmax gate, a router or selection bias) without defining them, and
// the grouped noaux_tc router that [vllmcpp]'s router dispatch names without
// defining it.  Reading: the published DeepSeek-V3 routing -
//   score s_e = softmax(L)_e (gate 0) or sigmoid(L_e) (gate 1),
//   selection key s_e + b_e (b the selection bias, zero when absent);
//   with n_group > 1 (grouped routing) the E experts form n_group groups of
//   E / n_group consecutive experts, a group's score is the sum of its two
//   largest keys (its one key for groups of one expert), the topk_group
//   groups with the largest scores are kept (the lower group index winning
//   a tie), and only the kept groups' experts can be picked;
//   the top-k keys among the pickable experts in rank order, the lower
//   index winning a tie,
//   weights from the unbiased scores of the picks, renormalised to sum to
//   one, times the routed scale: w_j = scale * s_j / sum_j' s_j'.
// For the softmax gate the full denominator cancels in the weights, so they
// are exp(L_j - m) / sum_j' exp(L_j' - m) with m the largest picked logit.
// Everything in fp64.
void variant_row(const float* L, int64_t E, int64_t k, int gate, const float* bias,
                 int64_t n_group, int64_t topk_group, double scale, int32_t* idx, double* w) {
  std::vector<double> s(E), key(E);
  if (gate == 1) {
    for (int64_t e = 0; e < E; ++e) s[e] = sigmoid((double)L[e]);
  } else {
    double m = (double)L[0];
    for (int64_t e = 1; e < E; ++e) m = std::max(m, (double)L[e]);
    double den = 0.0;
    for (int64_t e = 0; e < E; ++e) den += std::exp((double)L[e] - m);
    for (int64_t e = 0; e < E; ++e) s[e] = std::exp((double)L[e] - m) / den;
  }
  for (int64_t e = 0; e < E; ++e) key[e] = s[e] + (bias ? (double)bias[e] : 0.0);
  std::vector<char> pickable(E, 1);
  if (n_group > 1) {
    const int64_t gsz = E / n_group;
    std::vector<double> gscore(n_group);
    for (int64_t g = 0; g < n_group; ++g) {
      // the group's keys, largest first
      std::vector<double> kg(key.begin() + g * gsz, key.begin() + (g + 1) * gsz);
      std::sort(kg.begin(), kg.end(), [](double a, double b) { return a > b; });
      gscore[g] = gsz >= 2 ? kg[0] + kg[1] : kg[0];
    }
    std::vector<char> kept(n_group, 0);
    for (int64_t j = 0; j < topk_group; ++j) {
      int64_t best = -1;
      for (int64_t g = 0; g < n_group; ++g) {
        if (kept[g]) continue;
        if (best < 0 || gscore[g] > gscore[best]) best = g;  // strict: lower index keeps a tie
      }
      kept[best] = 1;
    }
    for (int64_t e = 0; e < E; ++e) pickable[e] = kept[e / gsz];
  }
  std::vector<char> taken(E, 0);
  for (int64_t j = 0; j < k; ++j) {
    int64_t best = -1;
    for (int64_t e = 0; e < E; ++e) {
      if (taken[e] || !pickable[e]) continue;
      if (best < 0 || key[e] > key[best]) best = e;
    }
    taken[best] = 1;
    idx[j] = (int32_t)best;
  }
  double den = 0.0;
  for (int64_t j = 0; j < k; ++j) den += s[idx[j]];
  for (int64_t j = 0; j < k; ++j) w[j] = scale * s[idx[j]] / den;
}

// One token row's routing: the plain softmax router (select_row,
// weights_row, then the optional top-p), or a variant, grouped or not
// (variant_row; top-p is not defined for variants and is ignored).  Returns
// the kept picks.  n_group <= 1 means no grouping.
int64_t route_row(const float* L, int64_t E, int64_t k, double scale, double top_p, int gate,
                  const float* bias, int64_t n_group, int64_t topk_group, int32_t* idx,
                  double* w) {
  if (gate == 0 && !bias && n_group <= 1) {
    select_row(L, E, k, idx);
    weights_row(L, idx, k, scale, w);
    return top_p_row(L, E, k, top_p, scale, idx, w);
  }
  variant_row(L, E, k, gate, bias, n_group, topk_group, scale, idx, w);
  return k;
}

}  // namespace

extern "C" {

// Threads used by oracle_layer's loop over token rows (0 = leave as is);
// returns the count now in effect.
int oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

double oracle_half_to_double(uint16_t h) { return half_to_double(h); }
double oracle_bf16_to_double(uint16_t b) { return bf16_to_double(b); }

// W[n][kk] = (nibble - 8) * scale, exact in fp64 (and in fp32: an fp16 scale
// times an integer in [-8, 7] needs at most 15 significant bits).
void oracle_dequant_int4(const uint8_t* q, const uint16_t* s, int64_t N, int64_t K, double* out) {
  for (int64_t n = 0; n < N; ++n)
    for (int64_t kk = 0; kk < K; ++kk) out[n * K + kk] = weight_int4(q, s, K, n, kk);
}

double oracle_e2m1_to_double(int nib) { return e2m1_to_double(nib); }
double oracle_e8m0_to_double(uint8_t e) { return e8m0_to_double(e); }

// W[n][kk] = e2m1(nibble) * 2^(e - 127) of one MXFP4 plane (q [N][K/2],
// s [N][K/32] ue8m0 bytes), exact in fp64.
void oracle_dequant_mxfp4(const uint8_t* q, const uint8_t* s, int64_t N, int64_t K, double* out) {
  for (int64_t n = 0; n < N; ++n)
    for (int64_t kk = 0; kk < K; ++kk) out[n * K + kk] = weight_mxfp4(q, s, K, n, kk);
}

// Router logits L[t][e] = sum_h x[t][h] * Wr[e][h] ([dasllama] routed-block
// commit: the router GEMM over the FFN-normed rows against the f32 router
// plane).  fp64 accumulation, rounded to fp32.  When gate_row is non-null the
// shared expert's gate logit a[t] = x[t].g is written as column E (the
// [dasllama] shared-expert decode commit computes that logit as an extra
// router row placed after the expert logits); out is then [T][E+1].
void oracle_router_logits(const uint16_t* x, const float* wr, const float* gate_row,
                          int64_t T, int64_t H, int64_t E, float* out) {
  const int64_t ld = E + (gate_row ? 1 : 0);
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t e = 0; e < ld; ++e) {
      const float* row = (e < E) ? wr + e * H : gate_row;
      double acc = 0.0;
      for (int64_t h = 0; h < H; ++h) acc += bf16_to_double(x[t * H + h]) * (double)row[h];
      out[t * ld + e] = (float)acc;
    }
  }
}

// Softmax -> top-k -> renormalise for every token row, then the optional
// expert top-p (top_p_row; top_p outside (0, 1) = off); or a router variant
// (gate 1 = sigmoid, bias [E] nullable, n_group > 1 grouped: variant_row).  idx [T][k]
// position-major in rank order (-1 for a pick top-p drops), w [T][k] rounded
// to fp32; w64 (nullable) receives the unrounded fp64 weights.
void oracle_router_topk(const float* logits, int64_t T, int64_t E, int64_t k, double route_scale,
                        double top_p, int gate, const float* bias, int64_t n_group,
                        int64_t topk_group, int32_t* idx, float* w, double* w64) {
  std::vector<double> wr(k);
  for (int64_t t = 0; t < T; ++t) {
    route_row(logits + t * E, E, k, route_scale, top_p, gate, bias, n_group, topk_group,
              idx + t * k, wr.data());
    for (int64_t j = 0; j < k; ++j) {
      w[t * k + j] = (float)wr[j];
      if (w64) w64[t * k + j] = wr[j];
    }
  }
}

// Token-to-expert permutation ([dasllama] routed-block commit: a per-expert
// count, an exclusive scan placing the buckets, the slot map in slot order).
// Slot s = t*k + j.  off[E+1] is the exclusive scan of the counts; within a
// bucket the slots appear in ascending slot order; row_of[s] is the row of
// slot s in the sorted order, so sorted[row_of[s]] == s.
// A pick outside [0, E) belongs to no bucket.  Reading: expert top-p (see
// top_p_row) leaves a dropped pick as index -1, and a dropped pick is routed
// nowhere, so it is counted in no bucket, takes no row (row_of[s] = -1) and
// off[E] counts the valid picks only; sorted holds those off[E] slots.
void oracle_permute(const int32_t* idx, int64_t T, int64_t k, int64_t E, int32_t* off,
                    int32_t* sorted, int32_t* row_of) {
  const int64_t S = T * k;
  auto valid = [&](int64_t s) { return idx[s] >= 0 && idx[s] < E; };
  std::vector<int64_t> cnt(E, 0);
  for (int64_t s = 0; s < S; ++s)
    if (valid(s)) cnt[idx[s]]++;
  off[0] = 0;
  for (int64_t e = 0; e < E; ++e) off[e + 1] = off[e] + (int32_t)cnt[e];
  std::vector<int64_t> cur(off, off + E);
  for (int64_t s = 0; s < S; ++s) {
    if (!valid(s)) {
      row_of[s] = -1;
      continue;
    }
    const int64_t r = cur[idx[s]]++;
    sorted[r] = (int32_t)s;
    row_of[s] = (int32_t)r;
  }
}

// One expert MLP on one activation row (fp64 in/out), for the tests.
// fmt: 0 = int4 (fp16 scales), 1 = MXFP4 (ue8m0 scales).
void oracle_expert_forward(const uint8_t* qg, const void* sg, const uint8_t* qu,
                           const void* su, const uint8_t* qd, const void* sd,
                           int64_t H, int64_t I, const double* x, double* h, double* o,
                           int fmt) {
  std::vector<double> hh(I);
  expert_forward(fmt, qg, sg, qu, su, qd, sd, H, I, x, h ? h : hh.data(), o);
}

// The combine folded into the residual step ([dasllama-fold]), for T rows:
//   r_out[t] = fp32(r[t] + y[t])                      (fp64 add, one rounding)
//   n_out[t] = bf16(r_out[t] * g / sqrt(mean_h r_out[t][h]^2 + eps))
// with y the layer's FFN row (shared row and slots already summed in order).
// Reading of the norm (the pages name it add+rms): RMS normalisation over
// the H features of the stored fp32 residual row, eps inside the square
// root, then the elementwise weight g of the next layer; computed in fp64
// and rounded once to bf16, the layer's activation format.  r_out may alias r.
void oracle_add_rmsnorm(const float* r, const float* y, const float* g, int64_t T, int64_t H,
                        double eps, float* r_out, uint16_t* n_out) {
  for (int64_t t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int64_t h = 0; h < H; ++h) {
      const float v = (float)((double)r[t * H + h] + (double)y[t * H + h]);
      r_out[t * H + h] = v;
      ss += (double)v * (double)v;
    }
    const double inv = 1.0 / std::sqrt(ss / (double)H + eps);
    for (int64_t h = 0; h < H; ++h)
      n_out[t * H + h] = double_to_bf16((double)r_out[t * H + h] * inv * (double)g[h]);
  }
}

uint16_t oracle_double_to_bf16(double v) { return double_to_bf16(v); }

// The residual step with the next layer's router folded in ([dasllama-fold]
// norms the row for the next layer; the vllm.cpp PR's closing hypotheses
// fold the router into the preceding kernel): oracle_add_rmsnorm, then the
// next layer's router logits of the bf16 normed row n_out, as
// oracle_router_logits computes them (fp64 sums of the exact products,
// rounded to fp32): logits[t][e] = sum_h n_out[t][h] * wr[e][h], [T][E].
// Reading: the router reads the row in the activation format the next
// layer receives (bf16), not the unrounded fp64 norm.
void oracle_add_rmsnorm_router(const float* r, const float* y, const float* g, int64_t T,
                               int64_t H, double eps, const float* wr, int64_t E, float* r_out,
                               uint16_t* n_out, float* logits) {
  oracle_add_rmsnorm(r, y, g, T, H, eps, r_out, n_out);
  oracle_router_logits(n_out, wr, nullptr, T, H, E, logits);
}

struct oracle_shape {
  int64_t T, H, E, k, I, SI;
  double route_scale;
  int64_t fmt;   // weight format of every plane: 0 = int4, 1 = MXFP4
  double top_p;  // expert top-p after the top-k (outside (0, 1) = off)
  int64_t gate;  // router score: 0 = softmax, 1 = sigmoid
  const float* bias;  // selection bias [E], or null
  int64_t n_group, topk_group;  // grouped routing (n_group <= 1: none)
};

// The whole layer for the token rows listed in `rows` (all T rows when rows is
// null; nrows = number of rows evaluated).  Steps, in order:
//   selection + weights from the given logits [T][E];
//   each selected expert's SwiGLU MLP on the token's activation row;
//   combine y[t] = [sigma(a_t) * shared(x_t)] + sum_j w_j * o_j, summed in
//   that order - the gated shared row first, then the slots in rank order
//   ([dasllama] combine-fold commit) - in fp64, rounded to fp32.
// The shared expert ([dasllama] shared-expert commits) is present when
// shared_q[0] is non-null; its gate logit is a_t = x_t . shared_gate in fp64;
// a null shared_gate means an ungated shared expert, added at weight one.
// Planes are stacked [E][N][K/2] / [E][N][K/32] (gate, up: N=I, K=H; down:
// N=H, K=I); shared planes are single [N][K/2] / [N][K/32] with I -> SI.
// Scales are fp16 bits (int4) or ue8m0 bytes (MXFP4), per sh->fmt.
// y is [nrows][H]; idx_out [nrows][k] and w_out [nrows][k] are nullable.
void oracle_layer(const oracle_shape* sh, const uint16_t* x, const float* logits,
                  const uint8_t* gq, const void* gs, const uint8_t* uq, const void* us,
                  const uint8_t* dq, const void* ds, const uint8_t* const* shared_q,
                  const void* const* shared_s, const float* shared_gate, const int32_t* rows,
                  int64_t nrows, float* y, int32_t* idx_out, float* w_out) {
  const int64_t H = sh->H, E = sh->E, k = sh->k, I = sh->I, SI = sh->SI;
  const int fmt = (int)sh->fmt;
  const bool has_shared = shared_q && shared_q[0];
  const int64_t gate_plane = I * (H / 2), gate_scales = I * (H / 32);
  const int64_t down_plane = H * (I / 2), down_scales = H * (I / 32);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t t = rows ? rows[r] : r;
    std::vector<double> xd(H), o(H), acc(H, 0.0), hbuf(std::max(I, SI));
    for (int64_t h = 0; h < H; ++h) xd[h] = bf16_to_double(x[t * H + h]);
    std::vector<int32_t> idx(k);
    std::vector<double> w(k);
    const int64_t kept = route_row(logits + t * E, E, k, sh->route_scale, sh->top_p,
                                   (int)sh->gate, sh->bias, sh->n_group, sh->topk_group,
                                   idx.data(), w.data());
    if (has_shared) {
      double gw = 1.0;
      if (shared_gate) {
        double a = 0.0;
        for (int64_t h = 0; h < H; ++h) a += xd[h] * (double)shared_gate[h];
        gw = sigmoid(a);
      }
      expert_forward(fmt, shared_q[0], shared_s[0], shared_q[1], shared_s[1], shared_q[2],
                     shared_s[2], H, SI, xd.data(), hbuf.data(), o.data());
      for (int64_t h = 0; h < H; ++h) acc[h] += gw * o[h];
    }
    for (int64_t j = 0; j < kept; ++j) {
      const int64_t e = idx[j];
      expert_forward(fmt, gq + e * gate_plane, scale_at(fmt, gs, e * gate_scales),
                     uq + e * gate_plane, scale_at(fmt, us, e * gate_scales),
                     dq + e * down_plane, scale_at(fmt, ds, e * down_scales), H, I,
                     xd.data(), hbuf.data(), o.data());
      for (int64_t h = 0; h < H; ++h) acc[h] += w[j] * o[h];
    }
    for (int64_t h = 0; h < H; ++h) y[r * H + h] = (float)acc[h];
    for (int64_t j = 0; j < k; ++j) {
      if (idx_out) idx_out[r * k + j] = idx[j];
      if (w_out) w_out[r * k + j] = (float)w[j];
    }
  }
}

}  // extern "C"
