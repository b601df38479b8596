// Streaming int4 GEMV for decode-sized buckets (a few tokens per expert).
//
// Sources: the colibri Vulkan-backend PR #418 (fused gate+up GEMV, the expert
// triple gate/up -> SiLU product -> down with the hidden row kept on the
// device, int4 offset-binary decode, one scale per 32 inputs applied to the
// packed-word partial) and the dasLLAMA vulkan PR #3988 GEMV lane split (a row
// gets 8, 16 or a whole subgroup of lanes by its block count, folded with an
// xor butterfly) and decode combine (routed slots weighted onto the output).
//
// Mapping on gfx950: a wave64 is cut into 64/LPR row lanes of LPR lanes; lane
// kl of a row lane owns the 32-input groups kl, kl+LPR, ... of every row it
// visits (GPL groups), so the activations it needs stay in VGPRs for the
// whole launch while the weight rows stream past with one 128-bit load per
// group (16 bytes = 32 nibbles = one scale group).  A wave walks `nit` row
// iterations in batches of RB rows held in two register sets: the loads of
// the next batch are issued before the current batch is reduced, so every
// wave keeps one to two batches of 16-byte loads in flight.  The grid is
// sized so that about 4096 waves cover the whole launch, which amortises each
// wave's serial prologue (bucket entry, token rows, activation registers).  The int4 -> bf16 decode and the exact dot products use
// v_dot2_f32_bf16 (see device.h); each group's fp32 partial is scaled once;
// the LPR-lane fold is a DPP add tree.  Gate/up rows are processed in pairs so
// SiLU(g)*u is formed in registers; the down launch multiplies by the slot's
// routing weight and adds into y with a hardware fp32 atomic.
#include "device.h"
#include "kernels.h"
#include "topk.h"

// Tuning constants (compile-time): waves the row iterations are spread over,
// the streaming-load hint, and the gate/up row batch at 3 groups per lane.
#ifndef MOE_GEMV_WAVES
#define MOE_GEMV_WAVES 2048
#endif
#ifndef MOE_GEMV_NT
#define MOE_GEMV_NT 1
#endif
#ifndef MOE_GEMV_RB3
#define MOE_GEMV_RB3 1
#endif

namespace moe {

namespace {

__device__ __forceinline__ uint4 load_w16(const void* p) {
#if MOE_GEMV_NT
  return load_stream16(p);
#else
  return *reinterpret_cast<const uint4*>(p);
#endif
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)v);
}

// Re-pair one aligned block of 8 bf16 activations (natural pairs n0..n3 =
// [x0,x1],[x2,x3],[x4,x5],[x6,x7]) into the operand order of q4_bf16_pairs
// ([x0,x4],[x1,x5],[x2,x6],[x3,x7]) and return the block's contribution to
// the offset correction, 136 * sum x.
__device__ __forceinline__ float pair_block(uint32_t n0, uint32_t n1, uint32_t n2, uint32_t n3,
                                            uint32_t* a) {
  a[0] = (n0 & 0xFFFFu) | (n2 << 16);
  a[1] = (n0 >> 16) | (n2 & 0xFFFF0000u);
  a[2] = (n1 & 0xFFFFu) | (n3 << 16);
  a[3] = (n1 >> 16) | (n3 & 0xFFFF0000u);
  const float sum = bf16_to_f32(n0 & 0xFFFF) + bf16_to_f32(n0 >> 16) + bf16_to_f32(n1 & 0xFFFF) +
                    bf16_to_f32(n1 >> 16) + bf16_to_f32(n2 & 0xFFFF) + bf16_to_f32(n2 >> 16) +
                    bf16_to_f32(n3 & 0xFFFF) + bf16_to_f32(n3 >> 16);
  return 136.0f * sum;
}

// Dot of one 32-input group (4 packed words) with a paired activation group.
__device__ __forceinline__ float dot_group(const Q4Pairs* p, const uint32_t* a) {
  float s = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    s = dot2_bf16(p[d].p0, a[4 * d + 0], s);
    s = dot2_bf16(p[d].p1, a[4 * d + 1], s);
    s = dot2_bf16(p[d].p2, a[4 * d + 2], s);
    s = dot2_bf16(p[d].p3, a[4 * d + 3], s);
  }
  return s;
}

struct BucketView {
  int e, r0, M;
};

__device__ __forceinline__ bool bucket_of(const Buckets& b, BucketView* v) {
  if (b.shared_T > 0) {
    if (blockIdx.y != 0) return false;
    v->e = 0;
    v->r0 = 0;
    v->M = b.shared_T;
    return true;
  }
  const int u = blockIdx.y;
  if (u >= b.sched[0]) return false;
  const int4 t = reinterpret_cast<const int4*>(b.sched + sched_touched_offset())[u];
  v->e = t.x;
  v->r0 = t.y;
  v->M = t.z;
  return true;
}

__device__ __forceinline__ int token_of(const Buckets& b, int r) {
  return b.shared_T > 0 ? r : b.sorted[r] / b.k;
}

// Bucket build of the fused small-batch routing (see RouteArgs), in LDS.
struct SmallRoute {
  int32_t pick[kFusedRouteMaxSlots];
  float wt[kFusedRouteMaxSlots];
  int32_t sorted[kFusedRouteMaxSlots];
  int32_t first[kFusedRouteMaxSlots];
  int4 bucket[kFusedRouteMaxSlots];
  int n_touched;
};

// Waves t < T take token t's top-k; then slot s (thread s) finds its row in
// the expert-major, slot-ascending order - #slots with a smaller expert plus
// #earlier slots with the same expert - exactly the permutation of the
// standalone kernels.  Every thread of the workgroup must call this.
template <int V>
__device__ void small_route(const RouteArgs& ra, int k, SmallRoute& sr) {
  const int tid = threadIdx.x, wave = tid >> 6;
  const bool publish = blockIdx.x == 0 && blockIdx.y == 0;
  const int S = ra.T * k;
  if (wave < ra.T)
    topk_wave<V>(ra.logits + (int64_t)wave * ra.ld, ra.E, k, ra.route_scale,
                 publish ? ra.idx + wave * k : nullptr, publish ? ra.w + wave * k : nullptr,
                 sr.pick + wave * k, sr.wt + wave * k);
  __syncthreads();
  int less = 0, rank = 0, first = 1, e = -1;
  if (tid < S) {
    e = sr.pick[tid];
    for (int s2 = 0; s2 < S; ++s2) {
      const int e2 = sr.pick[s2];
      less += e2 < e;
      if (s2 < tid && e2 == e) {
        ++rank;
        first = 0;
      }
    }
    sr.sorted[less + rank] = tid;
    sr.first[tid] = first;
    if (publish) {
      ra.sorted[less + rank] = tid;
      ra.row_of[tid] = less + rank;
    }
  }
  if (publish && tid < ra.E) {
    int o = 0;
    for (int s2 = 0; s2 < S; ++s2) o += sr.pick[s2] < tid;
    ra.off[tid] = o;
    if (tid == 0) ra.off[ra.E] = S;
  }
  __syncthreads();
  if (tid < S && first) {
    int u = 0, M = 0;
    for (int s2 = 0; s2 < S; ++s2) {
      u += sr.first[s2] && sr.pick[s2] < e;
      M += sr.pick[s2] == e;
    }
    sr.bucket[u] = make_int4(e, less, M, 0);
    if (publish) reinterpret_cast<int4*>(ra.sched + sched_touched_offset())[u] = sr.bucket[u];
  }
  if (tid == 0) {
    int n = 0;
    for (int s2 = 0; s2 < S; ++s2) n += sr.first[s2];
    sr.n_touched = n;
    if (publish) {
      ra.sched[0] = n;
      ra.sched[1] = 0;
    }
  }
  __syncthreads();
}

}  // namespace

template <int LPR, int GPL, int MT, int RB, int ROUTE_V>
__global__ __launch_bounds__(256) void gemv_gate_up_kernel(
    Buckets b, const uint16_t* __restrict__ x, int H, int I, const uint8_t* __restrict__ gq,
    const uint16_t* __restrict__ gs, const uint8_t* __restrict__ uq,
    const uint16_t* __restrict__ us, float* __restrict__ h, float* __restrict__ y_zero,
    int64_t y_elems, int nit, RouteArgs ra) {
  if (y_zero) {
    const int64_t nthr = (int64_t)gridDim.x * gridDim.y * blockDim.x;
    for (int64_t i = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
         i < y_elems; i += nthr)
      y_zero[i] = 0.f;
  }
  // ROUTE_V > 0: routing folded in (ROUTE_V logit registers per lane).
  __shared__ SmallRoute sr;
  BucketView bv;
  const int32_t* rows_sorted = b.sorted;
  if constexpr (ROUTE_V > 0) {
    small_route<ROUTE_V>(ra, b.k, sr);
    if ((int)blockIdx.y >= sr.n_touched) return;
    const int4 t = sr.bucket[blockIdx.y];
    bv.e = t.x;
    bv.r0 = t.y;
    bv.M = t.z;
    rows_sorted = sr.sorted;
  } else {
    if (!bucket_of(b, &bv)) return;
  }
  auto token_at = [&](int r) { return b.shared_T > 0 ? r : rows_sorted[r] / b.k; };

  constexpr int RPI = 64 / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = lane / LPR, kl = lane % LPR;
  const int G = H / 32;
  const int64_t pb = (int64_t)I * (H / 2), sb = (int64_t)I * G;
  const uint8_t* gqe = gq + bv.e * pb;
  const uint8_t* uqe = uq + bv.e * pb;
  const uint16_t* gse = gs + bv.e * sb;
  const uint16_t* use = us + bv.e * sb;
  const int row0 = (blockIdx.x * 4 + wave) * (nit * RPI) + rl;

  for (int m0 = 0; m0 < bv.M; m0 += MT) {
    const int nt = min(MT, bv.M - m0);
    // Row batches of RB rows, ping-ponged between two register sets so the
    // loads of the next batch are in flight while this one is reduced.
    struct Batch {
      uint4 g[RB][GPL], u[RB][GPL];
      uint32_t sg[RB][GPL], su[RB][GPL];  // fp16 bits, widened (keeps the batch in VGPRs)
    };
    auto load = [&](Batch& bt, int i0) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int n = row0 + (i0 + r) * RPI;
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) {
          const int g = kl + gi * LPR;
          if (n < I && g < G) {
            bt.g[r][gi] = load_w16(gqe + (int64_t)n * (H / 2) + 16 * g);
            bt.u[r][gi] = load_w16(uqe + (int64_t)n * (H / 2) + 16 * g);
            bt.sg[r][gi] = gse[(int64_t)n * G + g];
            bt.su[r][gi] = use[(int64_t)n * G + g];
          } else {
            bt.g[r][gi] = bt.u[r][gi] = make_uint4(0, 0, 0, 0);
            bt.sg[r][gi] = bt.su[r][gi] = 0;
          }
        }
      }
    };
    Batch A, B;
    load(A, 0);  // weights first: they do not wait for the activation prologue
    uint32_t xa[MT][GPL][16];
    float corr[MT][GPL];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint16_t* xr = x + (int64_t)token_at(bv.r0 + m0 + min(t, nt - 1)) * H;
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) {
        const int g = kl + gi * LPR;
        uint32_t nat[16];
        if (t < nt && g < G) {
          const uint4* src = reinterpret_cast<const uint4*>(xr + 32 * g);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint4 v = src[c];
            nat[4 * c] = v.x; nat[4 * c + 1] = v.y; nat[4 * c + 2] = v.z; nat[4 * c + 3] = v.w;
          }
        } else {
#pragma unroll
          for (int c = 0; c < 16; ++c) nat[c] = 0;
        }
        float cr = 0.f;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
          cr += pair_block(nat[4 * blk], nat[4 * blk + 1], nat[4 * blk + 2], nat[4 * blk + 3],
                           &xa[t][gi][4 * blk]);
        corr[t][gi] = cr;
      }
    }

    auto compute = [&](const Batch& bt, int i0) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int n = row0 + (i0 + r) * RPI;
        float ag[MT], au[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) ag[t] = au[t] = 0.f;
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) {
          const float fsg = half_bits_to_f32(bt.sg[r][gi]), fsu = half_bits_to_f32(bt.su[r][gi]);
          const Q4Pairs pg[4] = {q4_bf16_pairs(bt.g[r][gi].x), q4_bf16_pairs(bt.g[r][gi].y),
                                 q4_bf16_pairs(bt.g[r][gi].z), q4_bf16_pairs(bt.g[r][gi].w)};
          const Q4Pairs pu[4] = {q4_bf16_pairs(bt.u[r][gi].x), q4_bf16_pairs(bt.u[r][gi].y),
                                 q4_bf16_pairs(bt.u[r][gi].z), q4_bf16_pairs(bt.u[r][gi].w)};
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            if (t < nt) {
              ag[t] += fsg * (dot_group(pg, xa[t][gi]) - corr[t][gi]);
              au[t] += fsu * (dot_group(pu, xa[t][gi]) - corr[t][gi]);
            }
          }
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t < nt) {
            const float gsum = group_sum<LPR>(ag[t]);
            const float usum = group_sum<LPR>(au[t]);
            if (kl == LPR - 1 && n < I)
              h[(int64_t)(bv.r0 + m0 + t) * I + n] = gsum / (1.0f + __expf(-gsum)) * usum;
          }
        }
      }
    };
#pragma unroll 1
    for (int i0 = 0;;) {
      if (i0 + RB < nit) load(B, i0 + RB);
      compute(A, i0);
      i0 += RB;
      if (i0 >= nit) break;
      if (i0 + RB < nit) load(A, i0 + RB);
      compute(B, i0);
      i0 += RB;
      if (i0 >= nit) break;
    }
  }
}

template <int LPR, int GPL, int MT, int RB>
__global__ __launch_bounds__(256) void gemv_down_kernel(
    Buckets b, const float* __restrict__ h, int H, int I, const uint8_t* __restrict__ dq,
    const uint16_t* __restrict__ ds, const float* __restrict__ w,
    const float* __restrict__ gate_logit, int gate_ld, float* __restrict__ y, int nit) {
  BucketView bv;
  if (!bucket_of(b, &bv)) return;

  constexpr int RPI = 64 / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = lane / LPR, kl = lane % LPR;
  const int G = I / 32;
  const int64_t pb = (int64_t)H * (I / 2), sb = (int64_t)H * G;
  const uint8_t* dqe = dq + bv.e * pb;
  const uint16_t* dse = ds + bv.e * sb;
  const int row0 = (blockIdx.x * 4 + wave) * (nit * RPI) + rl;

  for (int m0 = 0; m0 < bv.M; m0 += MT) {
    const int nt = min(MT, bv.M - m0);
    struct Batch {
      uint4 d[RB][GPL];
      uint32_t sd[RB][GPL];  // fp16 bits, widened
    };
    auto load = [&](Batch& bt, int i0) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int n = row0 + (i0 + r) * RPI;
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) {
          const int g = kl + gi * LPR;
          if (n < H && g < G) {
            bt.d[r][gi] = load_w16(dqe + (int64_t)n * (I / 2) + 16 * g);
            bt.sd[r][gi] = dse[(int64_t)n * G + g];
          } else {
            bt.d[r][gi] = make_uint4(0, 0, 0, 0);
            bt.sd[r][gi] = 0;
          }
        }
      }
    };
    Batch A, B;
    load(A, 0);  // weights first: they do not wait for the activation prologue
    uint32_t xh[MT][GPL][16], xl[MT][GPL][16];
    float corr[MT][GPL], wt[MT];
    int tok[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int r = bv.r0 + m0 + min(t, nt - 1);
      if (b.shared_T > 0) {
        tok[t] = r;
        wt[t] = gate_logit ? sigmoidf_acc(gate_logit[(int64_t)r * gate_ld]) : 1.0f;
      } else {
        const int s = b.sorted[r];
        tok[t] = s / b.k;
        wt[t] = w[s];
      }
      const float* hr = h + (int64_t)r * I;
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) {
        const int g = kl + gi * LPR;
        float v[32];
        if (t < nt && g < G) {
          const float4* src = reinterpret_cast<const float4*>(hr + 32 * g);
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const float4 q = src[c];
            v[4 * c] = q.x; v[4 * c + 1] = q.y; v[4 * c + 2] = q.z; v[4 * c + 3] = q.w;
          }
        } else {
#pragma unroll
          for (int c = 0; c < 32; ++c) v[c] = 0.f;
        }
        // h = hi + lo with hi, lo bf16: hi + lo carries ~16 significant bits.
        uint32_t hi[16], lo[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const uint32_t h0 = f32_to_bf16_rne(v[2 * c]), h1 = f32_to_bf16_rne(v[2 * c + 1]);
          const uint32_t l0 = f32_to_bf16_rne(v[2 * c] - bf16_to_f32(h0));
          const uint32_t l1 = f32_to_bf16_rne(v[2 * c + 1] - bf16_to_f32(h1));
          hi[c] = pack2(h0, h1);
          lo[c] = pack2(l0, l1);
        }
        float cr = 0.f;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
          cr += pair_block(hi[4 * blk], hi[4 * blk + 1], hi[4 * blk + 2], hi[4 * blk + 3],
                           &xh[t][gi][4 * blk]);
          cr += pair_block(lo[4 * blk], lo[4 * blk + 1], lo[4 * blk + 2], lo[4 * blk + 3],
                           &xl[t][gi][4 * blk]);
        }
        corr[t][gi] = cr;
      }
    }

    auto compute = [&](const Batch& bt, int i0) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int n = row0 + (i0 + r) * RPI;
        float acc[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = 0.f;
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) {
          const float fsd = half_bits_to_f32(bt.sd[r][gi]);
          const Q4Pairs pd[4] = {q4_bf16_pairs(bt.d[r][gi].x), q4_bf16_pairs(bt.d[r][gi].y),
                                 q4_bf16_pairs(bt.d[r][gi].z), q4_bf16_pairs(bt.d[r][gi].w)};
#pragma unroll
          for (int t = 0; t < MT; ++t)
            if (t < nt)
              acc[t] += fsd * (dot_group(pd, xh[t][gi]) + dot_group(pd, xl[t][gi]) - corr[t][gi]);
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t < nt) {
            const float o = group_sum<LPR>(acc[t]);
            if (kl == LPR - 1 && n < H) unsafeAtomicAdd(&y[(int64_t)tok[t] * H + n], wt[t] * o);
          }
        }
      }
    };
#pragma unroll 1
    for (int i0 = 0;;) {
      if (i0 + RB < nit) load(B, i0 + RB);
      compute(A, i0);
      i0 += RB;
      if (i0 >= nit) break;
      if (i0 + RB < nit) load(A, i0 + RB);
      compute(B, i0);
      i0 += RB;
      if (i0 >= nit) break;
    }
  }
}

// ---------------------------------------------------------------------------
// Launch-shape selection: the fewest groups per lane first (LPR = the
// smallest power of two covering the row's groups, at most a whole wave), then
// as many tokens in registers as the VGPR budget allows, then the row batch.
// ---------------------------------------------------------------------------
namespace {

struct GemvShape {
  int lpr, gpl;
};

GemvShape pick_shape(int K) {
  const int G = K / 32;
  int lpr = 4;
  while (lpr < G && lpr < 64) lpr *= 2;
  return {lpr, (G + lpr - 1) / lpr};
}

int pow2_floor_min(int v, int cap) {
  int r = 1;
  while (r * 2 <= v && r * 2 <= cap) r *= 2;
  return r;
}

// Rows per load batch: 4 (down) or 2 (gate/up pairs) 16-byte loads per group
// column; two batches are in flight per wave.
constexpr int rb_for_gate_up(int gpl) { return gpl == 1 ? 4 : gpl == 2 ? 2 : MOE_GEMV_RB3; }
constexpr int rb_for_down(int gpl) { return gpl == 1 ? 4 : gpl == 2 ? 2 : 1; }

// Row iterations per wave: enough waves to fill the chip about twice
// (256 CUs x 8 waves), every wave streaming a multiple of its batch.
int rows_per_wave(int N, int rpi, int buckets, int rb) {
  const int64_t row_iters = (int64_t)((N + rpi - 1) / rpi) * buckets;
  int64_t nit = (row_iters + MOE_GEMV_WAVES - 1) / MOE_GEMV_WAVES;
  nit = (nit + rb - 1) / rb * rb;
  if (nit < rb) nit = rb;
  if (nit > 64) nit = 64;
  return (int)nit;
}

}  // namespace

bool gemv_supported(int K) { return K % 32 == 0 && K / 32 <= 4 * 64; }

#define MOE_GEMV_CASES(X) \
  X(4, 1) X(8, 1) X(16, 1) X(32, 1) X(64, 1) X(64, 2) X(64, 3) X(64, 4)

hipError_t launch_gemv_gate_up(const Buckets& b, int max_buckets, const uint16_t* x, int H,
                               int I, const uint8_t* gq, const uint16_t* gs,
                               const uint8_t* uq, const uint16_t* us, float* h, float* y_zero,
                               int64_t y_elems, const Launch& L, const RouteArgs* route) {
  const GemvShape sh = pick_shape(H);
  RouteArgs ra{};
  int rv = 0;  // logit registers per lane of the folded routing (0 = routing done earlier)
  if (route) {
    ra = *route;
    rv = (ra.E + 63) / 64;
    if (ra.T > kFusedRouteMaxT || ra.T * b.k > kFusedRouteMaxSlots || rv > 4)
      return hipErrorInvalidValue;
  }
  const int mt = pow2_floor_min(b.max_rows, sh.gpl == 1 ? 4 : 2);
  const int buckets = b.shared_T > 0 ? 1 : max_buckets;
  const int nit = rows_per_wave(I, 64 / sh.lpr, buckets, rb_for_gate_up(sh.gpl));
  const int rpb = 4 * nit * (64 / sh.lpr);
  dim3 grid((I + rpb - 1) / rpb, buckets);
#define GU(LP, GP, MTv, RV)                                                                        \
  MOE_LAUNCH(L, (gemv_gate_up_kernel<LP, GP, MTv, rb_for_gate_up(GP), RV>), grid, dim3(256), 0, b, \
             x, H, I, gq, gs, uq, us, h, y_zero, y_elems, nit, ra)
#define X(LP, GP)                                                                                  \
  if (sh.lpr == LP && sh.gpl == GP) {                                                              \
    if (rv > 0) {                                                                                  \
      switch (rv * 8 + mt) {                                                                       \
        case 9: GU(LP, GP, 1, 1); break;                                                           \
        case 10: GU(LP, GP, 2, 1); break;                                                          \
        case 17: GU(LP, GP, 1, 2); break;                                                          \
        case 18: GU(LP, GP, 2, 2); break;                                                          \
        case 25: GU(LP, GP, 1, 3); break;                                                          \
        case 26: GU(LP, GP, 2, 3); break;                                                          \
        case 33: GU(LP, GP, 1, 4); break;                                                          \
        case 34: GU(LP, GP, 2, 4); break;                                                          \
        default: if (GP == 1 && mt == 4) GU(LP, 1, 4, 4); else return hipErrorInvalidValue;       \
      }                                                                                            \
    } else {                                                                                       \
      switch (mt) {                                                                                \
        case 1: GU(LP, GP, 1, 0); break;                                                           \
        case 2: GU(LP, GP, 2, 0); break;                                                           \
        default: if (GP == 1) GU(LP, 1, 4, 0); break;                                              \
      }                                                                                            \
    }                                                                                              \
    return hipGetLastError();                                                                      \
  }
  MOE_GEMV_CASES(X)
#undef X
#undef GU
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_down(const Buckets& b, int max_buckets, const float* h, int H, int I,
                            const uint8_t* dq, const uint16_t* ds, const float* w,
                            const float* gate_logit, int gate_ld, float* y, const Launch& L) {
  const GemvShape sh = pick_shape(I);
  const int mt = pow2_floor_min(b.max_rows, sh.gpl == 1 ? 2 : 1);
  const int buckets = b.shared_T > 0 ? 1 : max_buckets;
  const int nit = rows_per_wave(H, 64 / sh.lpr, buckets, rb_for_down(sh.gpl));
  const int rpb = 4 * nit * (64 / sh.lpr);
  dim3 grid((H + rpb - 1) / rpb, buckets);
#define X(LP, GP)                                                                                  \
  if (sh.lpr == LP && sh.gpl == GP) {                                                              \
    constexpr int RBv = rb_for_down(GP);                                                           \
    switch (mt) {                                                                                  \
      case 1: MOE_LAUNCH(L, (gemv_down_kernel<LP, GP, 1, RBv>), grid, dim3(256), 0, b, h, H, I, dq, ds, w, gate_logit, gate_ld, y, nit); break; \
      default: if (GP == 1) MOE_LAUNCH(L, (gemv_down_kernel<LP, 1, 2, RBv>), grid, dim3(256), 0, b, h, H, I, dq, ds, w, gate_logit, gate_ld, y, nit); break; \
    }                                                                                              \
    return hipGetLastError();                                                                      \
  }
  MOE_GEMV_CASES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace moe
