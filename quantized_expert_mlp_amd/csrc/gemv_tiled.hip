// Streaming GEMV over tiled planes (moe_pack_weights' layout) for a handful
// of tokens, so that one packed copy of the weights serves decode as well as
// the grouped MFMA GEMM's prefill.  It computes what the row-layout GEMV does
// (the colibri Vulkan-backend PR #418 expert triple: fused gate+up, SiLU
// product, down with the routed slots weighted onto the output; int4 offset
// binary or the later fmt=7 MXFP4, one scale per 32 inputs), with its
// products, per-group scaling and routing prologue.
//
// A tiled block holds 32 rows x 64 inputs in one kilobyte, lane l's 16
// bytes being row l%32, scale group 2c + l/32 - one load per lane reads a
// block whole.  A workgroup of kTiledWaves waves owns one block row (32
// weight rows) of one bucket and splits its K steps (blocks) among them;
// each lane accumulates its row's partial sums over its half-groups, the two
// halves meet by a lane swap, the waves' partials through LDS in a fixed
// order.  The activation row of the pass (one token) is prepared
// once per workgroup in LDS in the form the dot routines take (the same
// nibble pairing and offset correction as the row-layout GEMV), and a lane
// reads its group's words from there at each step.
#include "gemv_impl.h"

namespace moe {

namespace {

#ifndef MOE_TILED_WAVES
#define MOE_TILED_WAVES 4  // waves per workgroup, each a share of the K blocks
#endif
#ifndef MOE_TILED_RB
#define MOE_TILED_RB 2  // K blocks per load batch (two batches in flight)
#endif
constexpr int kTiledWaves = MOE_TILED_WAVES;

// One prepared activation group: 16 words for the dot routines and the
// group's offset correction (zero for MXFP4).  80 bytes, 16-byte aligned.
struct TiledAct {
  uint4 w[4];
  float corr;
  float pad[3];
};

// Prepare groups [0, G) of MT activation rows (row t at src + rowoff(t)) into
// act[t*G + g]; BF16: bf16 rows (gate/up), else fp16 rows (down).
template <int MT, int FMT, bool BF16, typename RowOf>
__device__ __forceinline__ void tiled_stage(TiledAct* act, const uint16_t* src, int G, int nt,
                                            RowOf&& rowoff) {
  for (int i = threadIdx.x; i < MT * G; i += blockDim.x) {
    const int t = i / G, g = i - t * G;
    const uint4* p = reinterpret_cast<const uint4*>(src + rowoff(min(t, nt - 1)) + 32 * g);
    uint32_t nat[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 v = p[c];
      nat[4 * c] = v.x; nat[4 * c + 1] = v.y; nat[4 * c + 2] = v.z; nat[4 * c + 3] = v.w;
    }
    uint32_t o[16];
    float sum = 0.f;
    if constexpr (FMT == kFmtMxfp4) {
#pragma unroll
      for (int c = 0; c < 16; ++c) o[c] = BF16 ? bf16x2_to_f16x2(nat[c]) : nat[c];
    } else {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        pair_block(nat[4 * blk], nat[4 * blk + 1], nat[4 * blk + 2], nat[4 * blk + 3], &o[4 * blk]);
        sum += BF16 ? sum8_bf16(nat[4 * blk], nat[4 * blk + 1], nat[4 * blk + 2], nat[4 * blk + 3])
                    : sum8_f16(nat[4 * blk], nat[4 * blk + 1], nat[4 * blk + 2], nat[4 * blk + 3]);
      }
    }
    TiledAct& a = act[i];
#pragma unroll
    for (int c = 0; c < 4; ++c) a.w[c] = make_uint4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
    a.corr = FMT == kFmtMxfp4 ? 0.f : (BF16 ? 136.0f : 1032.0f) * sum;
  }
}

// The group dot of one lane's 16 weight bytes with a prepared group's words.
template <int FMT, bool BF16>
__device__ __forceinline__ float tiled_dot(uint4 w, const uint32_t (&x)[16], float corr) {
  if constexpr (FMT == kFmtMxfp4) return dot_group_mx(w, x);
  else if constexpr (BF16) return dot_group_bf16(w, x) - corr;
  else return dot_group_f16(w, x) - corr;
}

// K steps of one wave: P planes' blocks, RB steps per batch, two batches in
// flight; acc[p][t] gets sum over the wave's steps of scale * group dot.
// Unconditional loads: a step past the wave's range re-reads its last block
// (masked), so every load is counted in order.
template <int P, int MT, int RB, int FMT, bool BF16>
__device__ __forceinline__ void tiled_steps(const uint4* const (&q)[P],
                                            const typename GemvFmt<FMT>::S* const (&s)[P],
                                            const TiledAct* act, int G, int s0, int s1, int nt,
                                            float (&acc)[P][MT]) {
  using F = GemvFmt<FMT>;
  const int hf = (threadIdx.x & 63) >> 5;
  struct Batch {
    uint4 w[P][RB];
    uint32_t sc[P][RB];
  };
  const int last = s1 > s0 ? s1 - 1 : s0;
  auto load = [&](Batch& bt, int st) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int c = min(st + r, last);
#pragma unroll
      for (int p = 0; p < P; ++p) {
        bt.w[p][r] = load_w16(q[p] + (int64_t)c * 64);
        bt.sc[p][r] = s[p][(int64_t)c * 64];
      }
    }
  };
  // one token's group words at a time, shared by the P planes
  auto compute = [&](const Batch& bt, int st) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const bool live = st + r < s1;
      const int g = min(2 * (st + r) + hf, G - 1);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if (t < nt) {
          const TiledAct& a = act[t * G + g];
          uint32_t x[16];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint4 v = a.w[c];
            x[4 * c] = v.x; x[4 * c + 1] = v.y; x[4 * c + 2] = v.z; x[4 * c + 3] = v.w;
          }
          const float corr = a.corr;
#pragma unroll
          for (int p = 0; p < P; ++p) {
            const float d = F::scale(bt.sc[p][r]) * tiled_dot<FMT, BF16>(bt.w[p][r], x, corr);
            acc[p][t] += live ? d : 0.f;
          }
        }
      }
    }
  };
  Batch A, B;
  load(A, s0);
  int st = s0;
#pragma unroll 1
  for (; st + 2 * RB < s1; st += 2 * RB) {
    load(B, st + RB);
    compute(A, st);
    load(A, st + 2 * RB);
    compute(B, st + RB);
  }
  if (st + RB < s1) {
    load(B, st + RB);
    compute(A, st);
    compute(B, st + RB);
  } else {
    compute(A, st);
  }
}

// Sum of v over the two half-group lanes of a row (l and l ^ 32), then over
// the waves in a fixed order through red (kTiledWaves * 32 floats);
// the result is valid in wave 0's lanes 0..31.  Every thread calls.
__device__ __forceinline__ float tiled_reduce(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v += __shfl_xor(v, 32, 64);
  if (lane < 32) red[wave * 32 + lane] = v;
  __syncthreads();
  float s = 0.f;
  if (wave == 0 && lane < 32) {
#pragma unroll
    for (int w = 0; w < kTiledWaves; ++w) s += red[w * 32 + lane];
  }
  __syncthreads();
  return s;
}

template <int MT, int RB, int ROUTE_V, int FMT>
__global__ __launch_bounds__(64 * kTiledWaves) void gemv_tiled_gate_up_kernel(
    Buckets b, const uint16_t* __restrict__ x, int H, int I, const uint8_t* __restrict__ gq,
    const void* __restrict__ gs, const uint8_t* __restrict__ uq, const void* __restrict__ us,
    uint16_t* __restrict__ h, float* __restrict__ y_zero, int64_t y_elems, RouteArgs ra) {
  using SE = typename GemvFmt<FMT>::S;
  if (y_zero) {
    const int64_t nthr = (int64_t)gridDim.x * gridDim.y * blockDim.x;
    for (int64_t i = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
         i < y_elems; i += nthr)
      y_zero[i] = 0.f;
  }
  extern __shared__ __attribute__((aligned(16))) char tiled_lds[];
  __shared__ int32_t pick_lds[kFusedRouteMaxSlots];
  __shared__ float red[kTiledWaves * 32];
  TiledAct* act = reinterpret_cast<TiledAct*>(tiled_lds);
  BucketView bv;
  SmallRoute sr;
  if constexpr (ROUTE_V > 0) {
    small_route<ROUTE_V>(ra, b.k, pick_lds, sr);
    if ((int)blockIdx.y >= sr.n_touched) return;
    bv.e = sr.e;
    bv.r0 = sr.r0;
    bv.M = sr.M;
  } else {
    if (!bucket_of(b, &bv)) return;
  }
  auto token_at = [&](int r) {
    if (b.shared_T > 0) return r;
    if constexpr (ROUTE_V > 0)
      return (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(sr.pos == r)) / b.k;
    return load_uniform_i32(b.sorted + r) / b.k;
  };
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = H / 32, KS = H / 64, rg = blockIdx.x;
  const int64_t blocks = (int64_t)(I / 32) * KS;  // per expert
  const uint4* q[2] = {reinterpret_cast<const uint4*>(gq) + (bv.e * blocks + (int64_t)rg * KS) * 64 + lane,
                       reinterpret_cast<const uint4*>(uq) + (bv.e * blocks + (int64_t)rg * KS) * 64 + lane};
  const SE* s[2] = {static_cast<const SE*>(gs) + (bv.e * blocks + (int64_t)rg * KS) * 64 + lane,
                    static_cast<const SE*>(us) + (bv.e * blocks + (int64_t)rg * KS) * 64 + lane};
  const int s0 = KS * wave / kTiledWaves, s1 = KS * (wave + 1) / kTiledWaves;
  const int n = rg * 32 + (lane & 31);
  for (int m0 = 0; m0 < bv.M; m0 += MT) {
    const int nt = min(MT, bv.M - m0);
    // the previous pass's reads of act are done (tiled_reduce's barriers)
    int tok[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) tok[t] = token_at(bv.r0 + m0 + min(t, nt - 1));
    tiled_stage<MT, FMT, true>(act, x, G, nt, [&](int t) {
      int v = tok[0];
#pragma unroll
      for (int u = 1; u < MT; ++u) v = t == u ? tok[u] : v;
      return (int64_t)v * H;
    });
    __syncthreads();
    float acc[2][MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[0][t] = acc[1][t] = 0.f;
    tiled_steps<2, MT, RB, FMT, true>(q, s, act, G, s0, s1, nt, acc);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const float g = tiled_reduce(acc[0][t], red);
      const float u = tiled_reduce(acc[1][t], red);
      if (t < nt && wave == 0 && lane < 32 && n < I) {
        const _Float16 hv = (_Float16)(g / (1.0f + __expf(-g)) * u);
        h[(int64_t)(bv.r0 + m0 + t) * I + n] = __builtin_bit_cast(uint16_t, hv);
      }
    }
  }
}

template <int MT, int RB, int FMT>
__global__ __launch_bounds__(64 * kTiledWaves) void gemv_tiled_down_kernel(
    Buckets b, const uint16_t* __restrict__ hid, int H, int I, const uint8_t* __restrict__ dq,
    const void* __restrict__ ds, const float* __restrict__ w,
    const float* __restrict__ gate_logit, int gate_ld, float* __restrict__ y) {
  using SE = typename GemvFmt<FMT>::S;
  extern __shared__ __attribute__((aligned(16))) char tiled_lds[];
  __shared__ float red[kTiledWaves * 32];
  TiledAct* act = reinterpret_cast<TiledAct*>(tiled_lds);
  BucketView bv;
  if (!bucket_of(b, &bv)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = I / 32, KS = I / 64, rg = blockIdx.x;
  const int64_t blocks = (int64_t)(H / 32) * KS;
  const uint4* q[1] = {reinterpret_cast<const uint4*>(dq) + (bv.e * blocks + (int64_t)rg * KS) * 64 + lane};
  const SE* s[1] = {static_cast<const SE*>(ds) + (bv.e * blocks + (int64_t)rg * KS) * 64 + lane};
  const int s0 = KS * wave / kTiledWaves, s1 = KS * (wave + 1) / kTiledWaves;
  const int n = rg * 32 + (lane & 31);
  for (int m0 = 0; m0 < bv.M; m0 += MT) {
    const int nt = min(MT, bv.M - m0);
    tiled_stage<MT, FMT, false>(act, hid, G, nt,
                                [&](int t) { return (int64_t)(bv.r0 + m0 + t) * I; });
    __syncthreads();
    float acc[1][MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[0][t] = 0.f;
    tiled_steps<1, MT, RB, FMT, false>(q, s, act, G, s0, s1, nt, acc);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const float o = tiled_reduce(acc[0][t], red);
      if (t < nt && wave == 0 && lane < 32 && n < H) {
        const int r = bv.r0 + m0 + t;
        int tk;
        float wt;
        if (b.shared_T > 0) {
          tk = r;
          wt = gate_logit ? sigmoidf_acc(gate_logit[(int64_t)r * gate_ld]) : 1.0f;
        } else {
          const int sl = b.sorted[r];
          tk = sl / b.k;
          wt = w[sl];
        }
        unsafeAtomicAdd(&y[(int64_t)tk * H + n], wt * o);
      }
    }
  }
}

// One token per pass: a bucket of M rows streams its weights M times (the
// path serves a few tokens, whose buckets are mostly single rows); K steps
// per load batch.
constexpr int kTiledMT = 1, kTiledRB = MOE_TILED_RB;

size_t tiled_lds_bytes(int K, int mt) { return (size_t)mt * (K / 32) * sizeof(TiledAct); }

template <int FMT>
hipError_t tiled_gate_up_launch(const Buckets& b, int max_buckets, const uint16_t* x, int H, int I,
                                const uint8_t* gq, const void* gs, const uint8_t* uq,
                                const void* us, uint16_t* h, float* y_zero, int64_t y_elems,
                                const Launch& L, const RouteArgs* route) {
  RouteArgs ra{};
  int rv = 0;
  if (route) {
    ra = *route;
    rv = (ra.E + 63) / 64;
    if (ra.T > kFusedRouteMaxT || ra.T * b.k > kFusedRouteMaxSlots || rv > 4)
      return hipErrorInvalidValue;
  }
  const int buckets = b.shared_T > 0 ? 1 : max_buckets;
  const dim3 grid(I / 32, buckets);
  const size_t lds = tiled_lds_bytes(H, kTiledMT);
  if (lds > 48 * 1024) return hipErrorInvalidValue;
#define TG(RV)                                                                                   \
  MOE_LAUNCH(L, (gemv_tiled_gate_up_kernel<kTiledMT, kTiledRB, RV, FMT>), grid,                 \
             dim3(64 * kTiledWaves), lds, b, x, H, I, gq, gs, uq, us, h, y_zero, y_elems, ra)
  switch (rv) {
    case 0: TG(0); break;
    case 1: TG(1); break;
    case 2: TG(2); break;
    case 3: TG(3); break;
    case 4: TG(4); break;
    default: return hipErrorInvalidValue;
  }
#undef TG
  return hipGetLastError();
}

template <int FMT>
hipError_t tiled_down_launch(const Buckets& b, int max_buckets, const uint16_t* hid, int H, int I,
                             const uint8_t* dq, const void* ds, const float* w,
                             const float* gate_logit, int gate_ld, float* y, const Launch& L) {
  const int buckets = b.shared_T > 0 ? 1 : max_buckets;
  const dim3 grid(H / 32, buckets);
  const size_t lds = tiled_lds_bytes(I, kTiledMT);
  if (lds > 48 * 1024) return hipErrorInvalidValue;
  MOE_LAUNCH(L, (gemv_tiled_down_kernel<kTiledMT, kTiledRB, FMT>), grid, dim3(64 * kTiledWaves),
             lds, b, hid, H, I, dq, ds, w, gate_logit, gate_ld, y);
  return hipGetLastError();
}

}  // namespace

bool gemv_tiled_supported(int K) {
  return K % 64 == 0 && tiled_lds_bytes(K, kTiledMT) <= 48 * 1024;
}

hipError_t launch_gemv_tiled_gate_up(const Buckets& b, int max_buckets, const uint16_t* x, int H,
                                     int I, const uint8_t* gq, const void* gs, const uint8_t* uq,
                                     const void* us, uint16_t* h, float* y_zero, int64_t y_elems,
                                     int fmt, const Launch& L, const RouteArgs* route) {
  if (fmt == kFmtMxfp4)
    return tiled_gate_up_launch<kFmtMxfp4>(b, max_buckets, x, H, I, gq, gs, uq, us, h, y_zero,
                                           y_elems, L, route);
  return tiled_gate_up_launch<kFmtInt4>(b, max_buckets, x, H, I, gq, gs, uq, us, h, y_zero,
                                        y_elems, L, route);
}

hipError_t launch_gemv_tiled_down(const Buckets& b, int max_buckets, const uint16_t* h, int H,
                                  int I, const uint8_t* dq, const void* ds, const float* w,
                                  const float* gate_logit, int gate_ld, float* y, int fmt,
                                  const Launch& L) {
  if (fmt == kFmtMxfp4)
    return tiled_down_launch<kFmtMxfp4>(b, max_buckets, h, H, I, dq, ds, w, gate_logit, gate_ld,
                                        y, L);
  return tiled_down_launch<kFmtInt4>(b, max_buckets, h, H, I, dq, ds, w, gate_logit, gate_ld, y,
                                     L);
}

}  // namespace moe
