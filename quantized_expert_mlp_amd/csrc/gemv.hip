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
// group (16 bytes = 32 nibbles = one scale group).  The int4 -> bf16 decode
// and the exact dot products use v_dot2_f32_bf16 (see device.h); each group's
// fp32 partial is scaled once.  Gate/up rows are processed in pairs so SiLU(g)*u
// is formed in registers; the down launch multiplies by the slot's routing
// weight and adds into y with a hardware fp32 atomic.
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kNit = 4;  // row iterations per wave per block

__device__ __forceinline__ float half_bits_to_f32(uint16_t v) {
  return (float)__builtin_bit_cast(_Float16, v);
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
  v->e = b.sched[2 + u];
  v->r0 = b.off[v->e];
  v->M = b.off[v->e + 1] - v->r0;
  return true;
}

__device__ __forceinline__ int token_of(const Buckets& b, int r) {
  return b.shared_T > 0 ? r : b.sorted[r] / b.k;
}

}  // namespace

template <int LPR, int GPL, int MT>
__global__ __launch_bounds__(256) void gemv_gate_up_kernel(
    Buckets b, const uint16_t* __restrict__ x, int H, int I, const uint8_t* __restrict__ gq,
    const uint16_t* __restrict__ gs, const uint8_t* __restrict__ uq,
    const uint16_t* __restrict__ us, float* __restrict__ h, float* __restrict__ y_zero,
    int64_t y_elems) {
  if (y_zero) {
    const int64_t nthr = (int64_t)gridDim.x * gridDim.y * blockDim.x;
    for (int64_t i = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
         i < y_elems; i += nthr)
      y_zero[i] = 0.f;
  }
  BucketView bv;
  if (!bucket_of(b, &bv)) return;

  constexpr int RPI = 64 / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = lane / LPR, kl = lane % LPR;
  const int G = H / 32;
  const int64_t pb = (int64_t)I * (H / 2), sb = (int64_t)I * G;
  const uint8_t* gqe = gq + bv.e * pb;
  const uint8_t* uqe = uq + bv.e * pb;
  const uint16_t* gse = gs + bv.e * sb;
  const uint16_t* use = us + bv.e * sb;
  const int row0 = blockIdx.x * (4 * kNit * RPI) + wave * (kNit * RPI) + rl;

  for (int m0 = 0; m0 < bv.M; m0 += MT) {
    const int nt = min(MT, bv.M - m0);
    uint32_t xa[MT][GPL][16];
    float corr[MT][GPL];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint16_t* xr = x + (int64_t)token_of(b, bv.r0 + m0 + min(t, nt - 1)) * H;
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

    for (int it = 0; it < kNit; ++it) {
      const int n = row0 + it * RPI;
      const bool nv = n < I;
      float ag[MT], au[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) ag[t] = au[t] = 0.f;
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) {
        const int g = kl + gi * LPR;
        if (nv && g < G) {
          const uint4 wg = *reinterpret_cast<const uint4*>(gqe + (int64_t)n * (H / 2) + 16 * g);
          const uint4 wu = *reinterpret_cast<const uint4*>(uqe + (int64_t)n * (H / 2) + 16 * g);
          const float sg = half_bits_to_f32(gse[(int64_t)n * G + g]);
          const float su = half_bits_to_f32(use[(int64_t)n * G + g]);
          Q4Pairs pg[4] = {q4_bf16_pairs(wg.x), q4_bf16_pairs(wg.y), q4_bf16_pairs(wg.z),
                           q4_bf16_pairs(wg.w)};
          Q4Pairs pu[4] = {q4_bf16_pairs(wu.x), q4_bf16_pairs(wu.y), q4_bf16_pairs(wu.z),
                           q4_bf16_pairs(wu.w)};
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            if (t < nt) {
              ag[t] += sg * (dot_group(pg, xa[t][gi]) - corr[t][gi]);
              au[t] += su * (dot_group(pu, xa[t][gi]) - corr[t][gi]);
            }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        ag[t] = group_sum<LPR>(ag[t]);
        au[t] = group_sum<LPR>(au[t]);
      }
      if (kl == 0 && nv) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
          if (t < nt) {
            const float gv = ag[t];
            h[(int64_t)(bv.r0 + m0 + t) * I + n] = gv / (1.0f + __expf(-gv)) * au[t];
          }
      }
    }
  }
}

template <int LPR, int GPL, int MT>
__global__ __launch_bounds__(256) void gemv_down_kernel(
    Buckets b, const float* __restrict__ h, int H, int I, const uint8_t* __restrict__ dq,
    const uint16_t* __restrict__ ds, const float* __restrict__ w,
    const float* __restrict__ gate_logit, int gate_ld, float* __restrict__ y) {
  BucketView bv;
  if (!bucket_of(b, &bv)) return;

  constexpr int RPI = 64 / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = lane / LPR, kl = lane % LPR;
  const int G = I / 32;
  const int64_t pb = (int64_t)H * (I / 2), sb = (int64_t)H * G;
  const uint8_t* dqe = dq + bv.e * pb;
  const uint16_t* dse = ds + bv.e * sb;
  const int row0 = blockIdx.x * (4 * kNit * RPI) + wave * (kNit * RPI) + rl;

  for (int m0 = 0; m0 < bv.M; m0 += MT) {
    const int nt = min(MT, bv.M - m0);
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

    for (int it = 0; it < kNit; ++it) {
      const int n = row0 + it * RPI;
      const bool nv = n < H;
      float acc[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = 0.f;
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) {
        const int g = kl + gi * LPR;
        if (nv && g < G) {
          const uint4 wd = *reinterpret_cast<const uint4*>(dqe + (int64_t)n * (I / 2) + 16 * g);
          const float sd = half_bits_to_f32(dse[(int64_t)n * G + g]);
          Q4Pairs pd[4] = {q4_bf16_pairs(wd.x), q4_bf16_pairs(wd.y), q4_bf16_pairs(wd.z),
                           q4_bf16_pairs(wd.w)};
#pragma unroll
          for (int t = 0; t < MT; ++t)
            if (t < nt)
              acc[t] += sd * (dot_group(pd, xh[t][gi]) + dot_group(pd, xl[t][gi]) - corr[t][gi]);
        }
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = group_sum<LPR>(acc[t]);
      if (kl == 0 && nv) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
          if (t < nt) unsafeAtomicAdd(&y[(int64_t)tok[t] * H + n], wt[t] * acc[t]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launch-shape selection: the fewest groups per lane first (LPR = the
// smallest power of two covering the row's groups, at most a whole wave), then
// as many tokens in registers as the VGPR budget allows.
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

}  // namespace

bool gemv_supported(int K) { return K % 32 == 0 && K / 32 <= 4 * 64; }

#define MOE_GEMV_CASES(X) \
  X(4, 1) X(8, 1) X(16, 1) X(32, 1) X(64, 1) X(64, 2) X(64, 3) X(64, 4)

hipError_t launch_gemv_gate_up(const Buckets& b, int max_buckets, const uint16_t* x, int H,
                               int I, const uint8_t* gq, const uint16_t* gs,
                               const uint8_t* uq, const uint16_t* us, float* h, float* y_zero,
                               int64_t y_elems, hipStream_t st) {
  const GemvShape sh = pick_shape(H);
  const int max_tokens = b.max_rows;
  const int mt = pow2_floor_min(max_tokens, sh.gpl == 1 ? 8 : sh.gpl == 2 ? 4 : 2);
  const int rpb = 4 * kNit * (64 / sh.lpr);
  dim3 grid((I + rpb - 1) / rpb, b.shared_T > 0 ? 1 : max_buckets);
#define X(L, G)                                                                                  \
  if (sh.lpr == L && sh.gpl == G) {                                                              \
    switch (mt) {                                                                                \
      case 1: hipLaunchKernelGGL((gemv_gate_up_kernel<L, G, 1>), grid, dim3(256), 0, st, b, x, H, I, gq, gs, uq, us, h, y_zero, y_elems); break; \
      case 2: hipLaunchKernelGGL((gemv_gate_up_kernel<L, G, 2>), grid, dim3(256), 0, st, b, x, H, I, gq, gs, uq, us, h, y_zero, y_elems); break; \
      case 4: if (G <= 2) hipLaunchKernelGGL((gemv_gate_up_kernel<L, (G <= 2 ? G : 1), 4>), grid, dim3(256), 0, st, b, x, H, I, gq, gs, uq, us, h, y_zero, y_elems); break; \
      default: if (G == 1) hipLaunchKernelGGL((gemv_gate_up_kernel<L, 1, 8>), grid, dim3(256), 0, st, b, x, H, I, gq, gs, uq, us, h, y_zero, y_elems); break; \
    }                                                                                            \
    return hipGetLastError();                                                                    \
  }
  MOE_GEMV_CASES(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_down(const Buckets& b, int max_buckets, const float* h, int H, int I,
                            const uint8_t* dq, const uint16_t* ds, const float* w,
                            const float* gate_logit, int gate_ld, float* y, hipStream_t st) {
  const GemvShape sh = pick_shape(I);
  const int max_tokens = b.max_rows;
  const int mt = pow2_floor_min(max_tokens, sh.gpl == 1 ? 4 : sh.gpl == 2 ? 2 : 1);
  const int rpb = 4 * kNit * (64 / sh.lpr);
  dim3 grid((H + rpb - 1) / rpb, b.shared_T > 0 ? 1 : max_buckets);
#define X(L, G)                                                                                  \
  if (sh.lpr == L && sh.gpl == G) {                                                              \
    switch (mt) {                                                                                \
      case 1: hipLaunchKernelGGL((gemv_down_kernel<L, G, 1>), grid, dim3(256), 0, st, b, h, H, I, dq, ds, w, gate_logit, gate_ld, y); break; \
      case 2: if (G <= 2) hipLaunchKernelGGL((gemv_down_kernel<L, (G <= 2 ? G : 1), 2>), grid, dim3(256), 0, st, b, h, H, I, dq, ds, w, gate_logit, gate_ld, y); break; \
      default: if (G == 1) hipLaunchKernelGGL((gemv_down_kernel<L, 1, 4>), grid, dim3(256), 0, st, b, h, H, I, dq, ds, w, gate_logit, gate_ld, y); break; \
    }                                                                                            \
    return hipGetLastError();                                                                    \
  }
  MOE_GEMV_CASES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace moe
