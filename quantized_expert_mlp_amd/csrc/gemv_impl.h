// Streaming 4-bit GEMV for decode-sized buckets (a few tokens per expert):
// kernel templates over the weight format, instantiated by gemv.hip (int4)
// and gemv_mxfp4.hip (MXFP4), one translation unit per format.
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
// the next batch are issued before the current batch is reduced, and a
// wave's first batch is requested before its activation prologue.  When the
// group count allows (G % 8 == 0) a batch's scales - contiguous in memory -
// arrive as one 16-byte load per lane and are spread through a wave-private
// LDS slot, instead of one 2-byte load per lane, row and group.
//
// Arithmetic, int4: gate/up decodes nibbles to exact bf16 (128 + e) pairs and
// dots them with the bf16 activations (v_dot2_f32_bf16, exact products); down
// decodes to exact fp16 (1024 + e) pairs and dots them with the fp16 hidden
// row (v_dot2_f32_f16).  A per-group constant removes the offset.
// MXFP4 (the colibri PR's later fmt=7 comment: e2m1 nibbles, one ue8m0
// exponent per 32 inputs): each byte's two nibbles convert to their exact
// fp16 e2m1 pair with one packed fp4 conversion and dot with natural-order
// fp16 activation pairs (gate/up: the bf16 row converted once in the
// prologue); no offset.  Each group's fp32 partial is scaled once (fp16 scale,
// or 2^(e - 127) exactly in fp32); the LPR-lane fold is a DPP add tree.
// Gate/up rows are processed in pairs so SiLU(g)*u is formed in registers and
// stored as fp16; the down launch multiplies by the slot's routing weight and
// adds into y with a hardware fp32 atomic.
#pragma once

#include "device.h"
#include "kernels.h"
#include "topk.h"

// Tuning constants (compile-time): waves per token-register slot the row
// iterations are spread over, and the streaming-load hint.
#ifndef MOE_GEMV_WAVES
#define MOE_GEMV_WAVES 2048
#endif
#ifndef MOE_GEMV_WAVES_DOWN1
#define MOE_GEMV_WAVES_DOWN1 4096  // the down launch when buckets pass one token at a time
#endif
#ifndef MOE_GEMV_NT
#define MOE_GEMV_NT 1
#endif
#ifndef MOE_GEMV_WG_WAVES
#define MOE_GEMV_WG_WAVES 4  // waves per workgroup, gate/up (one routing prologue each)
#endif
#ifndef MOE_GEMV_WG_WAVES_DOWN
#define MOE_GEMV_WG_WAVES_DOWN 4  // waves per workgroup, down
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

// Re-pair one aligned block of 8 16-bit activations (natural pairs n0..n3 =
// [x0,x1],[x2,x3],[x4,x5],[x6,x7]) into the operand order of the decode
// ([x0,x4],[x1,x5],[x2,x6],[x3,x7]).
__device__ __forceinline__ void pair_block(uint32_t n0, uint32_t n1, uint32_t n2, uint32_t n3,
                                           uint32_t* a) {
  a[0] = (n0 & 0xFFFFu) | (n2 << 16);
  a[1] = (n0 >> 16) | (n2 & 0xFFFF0000u);
  a[2] = (n1 & 0xFFFFu) | (n3 << 16);
  a[3] = (n1 >> 16) | (n3 & 0xFFFF0000u);
}

__device__ __forceinline__ float sum8_bf16(uint32_t n0, uint32_t n1, uint32_t n2, uint32_t n3) {
  return bf16_to_f32(n0 & 0xFFFF) + bf16_to_f32(n0 >> 16) + bf16_to_f32(n1 & 0xFFFF) +
         bf16_to_f32(n1 >> 16) + bf16_to_f32(n2 & 0xFFFF) + bf16_to_f32(n2 >> 16) +
         bf16_to_f32(n3 & 0xFFFF) + bf16_to_f32(n3 >> 16);
}

__device__ __forceinline__ float sum8_f16(uint32_t n0, uint32_t n1, uint32_t n2, uint32_t n3) {
  return half_bits_to_f32(n0 & 0xFFFF) + half_bits_to_f32(n0 >> 16) +
         half_bits_to_f32(n1 & 0xFFFF) + half_bits_to_f32(n1 >> 16) +
         half_bits_to_f32(n2 & 0xFFFF) + half_bits_to_f32(n2 >> 16) +
         half_bits_to_f32(n3 & 0xFFFF) + half_bits_to_f32(n3 >> 16);
}

__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c,
                                false);
}

// sum_i (128 + e_i) x_i over one 32-input group (4 packed words).
__device__ __forceinline__ float dot_group_bf16(uint4 w, const uint32_t* a) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float s = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const Q4Pairs p = q4_bf16_pairs(ws[d]);
    s = dot2_bf16(p.p0, a[4 * d + 0], s);
    s = dot2_bf16(p.p1, a[4 * d + 1], s);
    s = dot2_bf16(p.p2, a[4 * d + 2], s);
    s = dot2_bf16(p.p3, a[4 * d + 3], s);
  }
  return s;
}

// sum_i (1024 + e_i) h_i over one 32-input group (4 packed words).
__device__ __forceinline__ float dot_group_f16(uint4 w, const uint32_t* a) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float s = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const Q4Pairs p = q4_f16_pairs(ws[d]);
    s = dot2_f16(p.p0, a[4 * d + 0], s);
    s = dot2_f16(p.p1, a[4 * d + 1], s);
    s = dot2_f16(p.p2, a[4 * d + 2], s);
    s = dot2_f16(p.p3, a[4 * d + 3], s);
  }
  return s;
}

// sum_i e2m1(e_i) a_i over one 32-input group (4 packed words) of MXFP4
// nibbles against fp16 activation pairs in natural order (a[j] holds inputs
// 2j, 2j+1): the fp16 e2m1 values are exact, so the products are exact in
// fp32.
__device__ __forceinline__ float dot_group_mx(uint4 w, const uint32_t* a) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float s = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    s = dot2_f16(e2m1_pair<0>(ws[d]), a[4 * d + 0], s);
    s = dot2_f16(e2m1_pair<1>(ws[d]), a[4 * d + 1], s);
    s = dot2_f16(e2m1_pair<2>(ws[d]), a[4 * d + 2], s);
    s = dot2_f16(e2m1_pair<3>(ws[d]), a[4 * d + 3], s);
  }
  return s;
}

// Two bf16 bit patterns (lo, hi halves of a) -> the fp16 pair, nearest even.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t a) {
  const f16x2_t h = {(_Float16)bf16_to_f32(a & 0xFFFFu), (_Float16)bf16_to_f32(a >> 16)};
  return __builtin_bit_cast(uint32_t, h);
}

// Weight-format traits: the scale element and its fp32 value.
template <int FMT>
struct GemvFmt;
template <>
struct GemvFmt<kFmtInt4> {
  using S = uint16_t;  // fp16 scale bits
  static __device__ __forceinline__ float scale(uint32_t v) { return half_bits_to_f32(v); }
};
template <>
struct GemvFmt<kFmtMxfp4> {
  using S = uint8_t;  // ue8m0 exponent
  static __device__ __forceinline__ float scale(uint32_t e) { return e8m0_f32(e); }
};

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
  // The entry is read together with the count (one memory round trip, not
  // two): blockIdx.y is below the launch's bucket bound, which the list's
  // capacity covers, and an entry past the count is never used.
  const int u = blockIdx.y;
  const int n = b.sched[0];
  const int4 t = reinterpret_cast<const int4*>(b.sched + sched_touched_offset())[u];
  v->e = t.x;
  v->r0 = t.y;
  v->M = t.z;
  return u < n;
}

// The fused small-batch routing (see RouteArgs), held in each wave's
// registers: lane s < T*k holds slot s's row (pos; -1 for a pick outside
// [0, E), which top-p writes as -1: it gets no row and no bucket); the
// bucket of this workgroup's blockIdx.y is wave-uniform, and blockIdx.y <
// n_touched says it exists.
struct SmallRoute {
  int pos;            // per lane
  int n_touched;      // uniform
  int e, r0, M;       // uniform: bucket blockIdx.y, when blockIdx.y < n_touched
};

// One token: the bucket of blockIdx.y is pick j = k - 1 - blockIdx.y, its
// one row is row j (slot j), so a workgroup needs only the first j + 1
// arg-max rounds (with the plain softmax router and no top-p; all k
// otherwise) and every wave takes them itself - no LDS, no barrier.  The
// down launch reads buckets u < (valid picks) as pick u: top-p's dropped
// picks are a suffix.  Workgroup (0,0) runs all k, forms the weights and publishes
// the picks, slot order, row_of and the bucket list for the down launch
// (the expert offsets are not formed: nothing reads them on this path).
//
// More tokens: wave t < T takes token t's top-k and the picks pass through
// LDS; rows are expert-major and slot-ascending, the permutation of the
// standalone kernels.  Every wave, from the S = T*k picks in its lanes,
// counts for slot s the valid slots with a smaller expert (less), the
// earlier ones with the same expert (rank) and all with the same expert
// (M): row = less + rank, and the slot with rank 0 opens its expert's
// bucket, whose index is the number of distinct experts below it.
// Workgroup (0,0) publishes the picks and weights, the permutation, the
// expert offsets and the bucket list.
//
// Every thread of the workgroup must call this.
template <int V>
__device__ void small_route(const RouteArgs& ra, int k, int32_t* pick_lds, SmallRoute& sr) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool publish = blockIdx.x == 0 && blockIdx.y == 0;
  auto valid = [&](int e2) { return e2 >= 0 && e2 < ra.E; };
  int e = -1;
  if (ra.T == 1) {  // uniform over the launch
    // the first-dispatched workgroups (low blockIdx.y), which the hardware
    // favours, take the picks decided last
    const int j = k - 1 - (int)blockIdx.y;
    const bool pw = publish && wave == 0;
    topk_group<V, 64>(ra.logits, ra.ld, 1, 0, ra.E, k, ra.rs, pw ? ra.idx : nullptr,
                      pw ? ra.w : nullptr, nullptr, nullptr, 0, pw, &e,
                      publish ? k : max(j + 1, 1));
    const int pj = j >= 0 ? __builtin_amdgcn_readlane(e, j) : -1;
    const bool mine = lane < k && valid(e);
    const int n_valid = __builtin_popcountll(__builtin_amdgcn_ballot_w64(mine));  // whole wave
    sr.pos = mine ? lane : -1;
    sr.n_touched = (int)blockIdx.y + (valid(pj) ? 1 : 0);
    sr.e = pj;
    sr.r0 = j;
    sr.M = 1;
    if (pw) {
      if (lane < k) {
        if (mine) {
          ra.sorted[lane] = lane;
          reinterpret_cast<int4*>(ra.sched + sched_touched_offset())[lane] = make_int4(e, lane, 1, 0);
        }
        ra.row_of[lane] = mine ? lane : -1;
      }
      if (lane == 0) {
        ra.sched[0] = n_valid;
        ra.sched[1] = 0;
      }
    }
    return;
  }
  const int S = ra.T * k;
  if (wave < ra.T)
    topk_group<V, 64>(ra.logits, ra.ld, ra.T, wave, ra.E, k, ra.rs, publish ? ra.idx : nullptr,
                      publish ? ra.w : nullptr, pick_lds, nullptr, 0, publish);
  __syncthreads();
  e = lane < S ? pick_lds[lane] : -1;
  int less = 0, rank = 0, M = 0;
  for (int s2 = 0; s2 < S; ++s2) {
    const int e2 = __builtin_amdgcn_readlane(e, s2);
    if (valid(e2)) {  // uniform
      less += e2 < e;
      M += e2 == e;
      rank += (e2 == e) & (s2 < lane);
    }
  }
  const bool mine = lane < S && valid(e);
  const bool first = mine && rank == 0;
  const uint64_t opens = __builtin_amdgcn_ballot_w64(first);
  int u = 0;  // distinct experts below e
  for (uint64_t m = opens; m != 0; m &= m - 1)
    u += __builtin_amdgcn_readlane(e, (int)__builtin_ctzll(m)) < e;
  sr.pos = mine ? less + rank : -1;
  sr.n_touched = __builtin_popcountll(opens);
  const uint64_t here = __builtin_amdgcn_ballot_w64(first && u == (int)blockIdx.y);
  sr.e = sr.r0 = sr.M = 0;
  if (here != 0) {
    const int s = (int)__builtin_ctzll(here);
    sr.e = __builtin_amdgcn_readlane(e, s);
    sr.r0 = __builtin_amdgcn_readlane(less, s);
    sr.M = __builtin_amdgcn_readlane(M, s);
  }
  if (publish) {
    if (wave == 0) {
      if (lane < S) {
        if (mine) ra.sorted[less + rank] = lane;
        ra.row_of[lane] = mine ? less + rank : -1;
      }
      if (first) reinterpret_cast<int4*>(ra.sched + sched_touched_offset())[u] = make_int4(e, less, M, 0);
      if (lane == 0) {
        ra.sched[0] = sr.n_touched;
        ra.sched[1] = 0;
      }
    }
    // expert offsets: thread x < E counts the valid slots below expert x
    for (int x = tid; x <= ra.E; x += blockDim.x) {
      int o = 0;
      for (int s2 = 0; s2 < S; ++s2) {
        const int e2 = __builtin_amdgcn_readlane(e, s2);
        o += valid(e2) && (x == ra.E || e2 < x);
      }
      ra.off[x] = o;
    }
  }
}

// One row batch's scales for P planes, staged through a wave-private LDS slot.
// Rows n0 .. n0 + RB*RPI - 1 of a plane are contiguous (RB*RPI*G scales of SB
// bytes = at most 512 bytes), so lane c < P * chunks loads 16-byte chunk
// c % chunks of plane c / chunks.  Needs G * SB % 16 == 0 (16-byte aligned
// chunk starts).  Lanes read words other lanes wrote, so the staging is
// bracketed by wave-level syncs (wave_lds_sync).
template <int P, int RB, int RPI, int SB>
struct ScaleStage {
  static constexpr int kMaxPlaneBytes = 512;
  uint4 v;
  // Every lane loads (no branch around the load, so the compiler's wait
  // counts stay exact): lanes past the batch's chunks, and chunks of rows
  // past N, re-read the plane's last chunk; stage() publishes only the
  // batch's own chunks and rows past N are never stored.
  template <typename T>
  __device__ __forceinline__ void load(const T* const* sp, int n0, int N, int G) {
    const int lane = threadIdx.x & 63;
    const int pbytes = RB * RPI * G * SB, chunks = pbytes / 16;
    const int p = lane / chunks, j = lane - p * chunks;
    const int64_t last = (int64_t)N * G * SB - 16;
    int64_t at = (int64_t)n0 * G * SB + 16 * j;
    at = at < last ? at : last;
    const u32x4_t w = load_global16(reinterpret_cast<const char*>(sp[p < P ? p : P - 1]) + at);
    v = make_uint4(w[0], w[1], w[2], w[3]);
  }
  // Publish this batch's chunks; the slot's previous contents (read by other
  // lanes for the previous batch) are overwritten only after those reads.
  __device__ __forceinline__ void stage(uint32_t* slot, int G) const {
    const int lane = threadIdx.x & 63;
    wave_lds_sync();
    if (lane < P * (RB * RPI * G * SB / 16)) {
      slot[4 * lane + 0] = v.x;
      slot[4 * lane + 1] = v.y;
      slot[4 * lane + 2] = v.z;
      slot[4 * lane + 3] = v.w;
    }
    wave_lds_sync();
  }
  // Bits of the scale of (plane, row in batch, group).
  static __device__ __forceinline__ uint32_t get(const uint32_t* slot, int p, int rr, int g,
                                                 int G) {
    const int i = p * (RB * RPI * G) + rr * G + g;
    if constexpr (SB == 2) return (slot[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
    else return (slot[i >> 2] >> (8 * (i & 3))) & 0xFFu;
  }
};

}  // namespace

constexpr int kGuWaves = MOE_GEMV_WG_WAVES, kDnWaves = MOE_GEMV_WG_WAVES_DOWN;
// the fused routing gives thread e expert e's offset (E <= 256) and wave t token t
static_assert(kGuWaves >= 4 && kGuWaves <= 16 && kDnWaves >= 1 && kDnWaves <= 16, "waves");

template <int LPR, int GPL, int MT, int RB, int ROUTE_V, bool SLDS, int FMT>

__global__ __launch_bounds__(64 * kGuWaves) void gemv_gate_up_kernel(
    Buckets b, const uint16_t* __restrict__ x, int H, int I, const uint8_t* __restrict__ gq,
    const void* __restrict__ gs, const uint8_t* __restrict__ uq, const void* __restrict__ us,
    uint16_t* __restrict__ h, float* __restrict__ y_zero, int64_t y_elems, int nit,
    RouteArgs ra) {
  using F = GemvFmt<FMT>;
  using SE = typename F::S;
  if (y_zero) {
    const int64_t nthr = (int64_t)gridDim.x * gridDim.y * blockDim.x;
    for (int64_t i = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
         i < y_elems; i += nthr)
      y_zero[i] = 0.f;
  }
  // ROUTE_V > 0: routing folded in (ROUTE_V logit registers per lane).
  __shared__ int32_t pick_lds[kFusedRouteMaxSlots];
  __shared__ uint32_t sslot[kGuWaves][ScaleStage<2, RB, 64 / LPR, 2>::kMaxPlaneBytes * 2 / 4];
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
  // the token of bucket row r (wave-uniform; with the fused routing the slot
  // whose row is r, from the lanes' rows, else a scalar load)
  auto token_at = [&](int r) {
    if (b.shared_T > 0) return r;
    if constexpr (ROUTE_V > 0)
      return (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(sr.pos == r)) / b.k;
    return load_uniform_i32(b.sorted + r) / b.k;
  };

  constexpr int RPI = 64 / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = lane / LPR, kl = lane % LPR;
  const int G = H / 32;
  const int64_t pb = (int64_t)I * (H / 2), sb = (int64_t)I * G;
  const uint8_t* gqe = gq + bv.e * pb;
  const uint8_t* uqe = uq + bv.e * pb;
  const SE* spl[2] = {static_cast<const SE*>(gs) + bv.e * sb,
                      static_cast<const SE*>(us) + bv.e * sb};
  const int rbase = (blockIdx.x * kGuWaves + wave) * (nit * RPI);  // first row of the wave
  const int row0 = rbase + rl;
  uint32_t* slot = sslot[wave];
  using SS = ScaleStage<2, RB, RPI, (int)sizeof(SE)>;

  for (int m0 = 0; m0 < bv.M; m0 += MT) {
    const int nt = min(MT, bv.M - m0);
    // Row batches of RB rows, ping-ponged between two register sets.
    struct Batch {
      uint4 g[RB][GPL], u[RB][GPL];
      uint32_t sg[RB][GPL], su[RB][GPL];  // per-lane scale bits when !SLDS
      SS sc;                              // staged scales when SLDS
    };
    // Unconditional loads (exact wait counts, so the next batch stays in
    // flight while this one is reduced): rows past I re-read row I - 1
    // (never stored), groups past G re-read group G - 1 (masked in compute).
    auto load = [&](Batch& bt, int i0) {
      if constexpr (SLDS) bt.sc.load(spl, rbase + i0 * RPI, I, G);
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int n = min(row0 + (i0 + r) * RPI, I - 1);
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) {
          const int g = min(kl + gi * LPR, G - 1);
          bt.g[r][gi] = load_w16(gqe + (int64_t)n * (H / 2) + 16 * g);
          bt.u[r][gi] = load_w16(uqe + (int64_t)n * (H / 2) + 16 * g);
          if constexpr (!SLDS) {
            bt.sg[r][gi] = spl[0][(int64_t)n * G + g];
            bt.su[r][gi] = spl[1][(int64_t)n * G + g];
          }
        }
      }
    };
    // The activation rows are loaded first and the first weight batch right
    // after them: loads complete in order, so waiting for the activations
    // leaves the weights in flight while the activations are prepared.
    // Unconditional loads (a clamped group), zeroed where they are not this
    // lane's: no branch for the compiler's wait counting.
    uint32_t xa[MT][GPL][16];
    float corr[MT][GPL];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint16_t* xr = x + (int64_t)token_at(bv.r0 + m0 + min(t, nt - 1)) * H;
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) {
        const uint4* src = reinterpret_cast<const uint4*>(xr + 32 * min(kl + gi * LPR, G - 1));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint4 v = src[c];
          xa[t][gi][4 * c] = v.x; xa[t][gi][4 * c + 1] = v.y;
          xa[t][gi][4 * c + 2] = v.z; xa[t][gi][4 * c + 3] = v.w;
        }
      }
    }
    Batch A, B;
    __builtin_amdgcn_sched_barrier(0);  // keep the activation loads ahead of the weights
    load(A, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) {
        const bool own = t < nt && kl + gi * LPR < G;
        uint32_t nat[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) nat[c] = own ? xa[t][gi][c] : 0u;
        float sum = 0.f;
        if constexpr (FMT == kFmtMxfp4) {
          // natural-order fp16 pairs (the MXFP4 decode yields natural pairs)
#pragma unroll
          for (int c = 0; c < 16; ++c) xa[t][gi][c] = bf16x2_to_f16x2(nat[c]);
        } else {
#pragma unroll
          for (int blk = 0; blk < 4; ++blk) {
            pair_block(nat[4 * blk], nat[4 * blk + 1], nat[4 * blk + 2], nat[4 * blk + 3],
                       &xa[t][gi][4 * blk]);
            sum += sum8_bf16(nat[4 * blk], nat[4 * blk + 1], nat[4 * blk + 2], nat[4 * blk + 3]);
          }
        }
        corr[t][gi] = 136.0f * sum;
      }
    }

    auto compute = [&](const Batch& bt, int i0) {
      if constexpr (SLDS) bt.sc.stage(slot, G);
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int n = row0 + (i0 + r) * RPI;
        float ag[MT], au[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) ag[t] = au[t] = 0.f;
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) {
          const int g = kl + gi * LPR;
          uint32_t sgb, sub;
          if constexpr (SLDS) {
            const int gg = g < G ? g : 0;
            sgb = SS::get(slot, 0, r * RPI + rl, gg, G);
            sub = SS::get(slot, 1, r * RPI + rl, gg, G);
          } else {
            sgb = bt.sg[r][gi];
            sub = bt.su[r][gi];
          }
          const float fsg = F::scale(sgb), fsu = F::scale(sub);
          const bool live = g < G;
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            if (t < nt) {
              float dg, du;
              if constexpr (FMT == kFmtMxfp4) {
                dg = fsg * dot_group_mx(bt.g[r][gi], xa[t][gi]);
                du = fsu * dot_group_mx(bt.u[r][gi], xa[t][gi]);
              } else {
                dg = fsg * (dot_group_bf16(bt.g[r][gi], xa[t][gi]) - corr[t][gi]);
                du = fsu * (dot_group_bf16(bt.u[r][gi], xa[t][gi]) - corr[t][gi]);
              }
              ag[t] += live ? dg : 0.f;
              au[t] += live ? du : 0.f;
            }
          }
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t < nt) {
            const float gsum = group_sum<LPR>(ag[t]);
            const float usum = group_sum<LPR>(au[t]);
            if (kl == LPR - 1 && n < I) {
              const _Float16 hv = (_Float16)(gsum / (1.0f + __expf(-gsum)) * usum);
              h[(int64_t)(bv.r0 + m0 + t) * I + n] = __builtin_bit_cast(uint16_t, hv);
            }
          }
        }
      }
    };
    // Batches i0, i0 + RB, ... (nit a multiple of RB): the loop body's
    // loads are all in range, the last one or two batches are peeled, so
    // no load sits behind a branch and each reduction waits only for its
    // own batch while the next one is in flight.
    int i0 = 0;
#pragma unroll 1
    for (; i0 + 2 * RB < nit; i0 += 2 * RB) {
      load(B, i0 + RB);
      compute(A, i0);
      load(A, i0 + 2 * RB);
      compute(B, i0 + RB);
    }
    if (i0 + RB < nit) {
      load(B, i0 + RB);
      compute(A, i0);
      compute(B, i0 + RB);
    } else {
      compute(A, i0);
    }
  }
}

template <int LPR, int GPL, int MT, int RB, bool SLDS, int FMT>
__global__ __launch_bounds__(64 * kDnWaves) void gemv_down_kernel(
    Buckets b, const uint16_t* __restrict__ h, int H, int I, const uint8_t* __restrict__ dq,
    const void* __restrict__ ds, const float* __restrict__ w,
    const float* __restrict__ gate_logit, int gate_ld, float* __restrict__ y, int nit) {
  using F = GemvFmt<FMT>;
  using SE = typename F::S;
  __shared__ uint32_t sslot[kDnWaves][ScaleStage<1, RB, 64 / LPR, 2>::kMaxPlaneBytes / 4];
  BucketView bv;
  if (!bucket_of(b, &bv)) return;

  constexpr int RPI = 64 / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = lane / LPR, kl = lane % LPR;
  const int G = I / 32;
  const int64_t pb = (int64_t)H * (I / 2), sb = (int64_t)H * G;
  const uint8_t* dqe = dq + bv.e * pb;
  const SE* spl[1] = {static_cast<const SE*>(ds) + bv.e * sb};
  const int rbase = (blockIdx.x * kDnWaves + wave) * (nit * RPI);
  const int row0 = rbase + rl;
  uint32_t* slot = sslot[wave];
  using SS = ScaleStage<1, RB, RPI, (int)sizeof(SE)>;

  for (int m0 = 0; m0 < bv.M; m0 += MT) {
    const int nt = min(MT, bv.M - m0);
    struct Batch {
      uint4 d[RB][GPL];
      uint32_t sd[RB][GPL];  // per-lane scale bits when !SLDS
      SS sc;
    };
    // Unconditional loads, as in the gate/up kernel: rows past H re-read row
    // H - 1 (never stored), groups past G re-read group G - 1 (masked).
    auto load = [&](Batch& bt, int i0) {
      if constexpr (SLDS) bt.sc.load(spl, rbase + i0 * RPI, H, G);
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int n = min(row0 + (i0 + r) * RPI, H - 1);
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) {
          const int g = min(kl + gi * LPR, G - 1);
          bt.d[r][gi] = load_w16(dqe + (int64_t)n * (I / 2) + 16 * g);
          if constexpr (!SLDS) bt.sd[r][gi] = spl[0][(int64_t)n * G + g];
        }
      }
    };
    // Activations (the hidden rows) first, then the first weight batch, as in
    // the gate/up kernel; the token and combine weight of each row are
    // wave-uniform scalar loads, counted apart from the vector loads.
    uint32_t xa[MT][GPL][16];
    float corr[MT][GPL], wt[MT];
    int tok[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int r = bv.r0 + m0 + min(t, nt - 1);
      const uint16_t* hr = h + (int64_t)r * I;
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) {
        const uint4* src = reinterpret_cast<const uint4*>(hr + 32 * min(kl + gi * LPR, G - 1));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint4 v = src[c];
          xa[t][gi][4 * c] = v.x; xa[t][gi][4 * c + 1] = v.y;
          xa[t][gi][4 * c + 2] = v.z; xa[t][gi][4 * c + 3] = v.w;
        }
      }
    }
    Batch A, B;
    __builtin_amdgcn_sched_barrier(0);  // keep the activation loads ahead of the weights
    load(A, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int r = bv.r0 + m0 + min(t, nt - 1);
      if (b.shared_T > 0) {
        tok[t] = r;
        wt[t] = gate_logit ? sigmoidf_acc(load_uniform_f32(gate_logit + (int64_t)r * gate_ld))
                           : 1.0f;
      } else {
        const int s = load_uniform_i32(b.sorted + r);
        tok[t] = s / b.k;
        wt[t] = load_uniform_f32(w + s);
      }
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) {
        const bool own = t < nt && kl + gi * LPR < G;
        uint32_t nat[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) nat[c] = own ? xa[t][gi][c] : 0u;
        float sum = 0.f;
        if constexpr (FMT == kFmtMxfp4) {
#pragma unroll
          for (int c = 0; c < 16; ++c) xa[t][gi][c] = nat[c];  // natural-order fp16 pairs
        } else {
#pragma unroll
          for (int blk = 0; blk < 4; ++blk) {
            pair_block(nat[4 * blk], nat[4 * blk + 1], nat[4 * blk + 2], nat[4 * blk + 3],
                       &xa[t][gi][4 * blk]);
            sum += sum8_f16(nat[4 * blk], nat[4 * blk + 1], nat[4 * blk + 2], nat[4 * blk + 3]);
          }
        }
        corr[t][gi] = 1032.0f * sum;
      }
    }

    auto compute = [&](const Batch& bt, int i0) {
      if constexpr (SLDS) bt.sc.stage(slot, G);
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int n = row0 + (i0 + r) * RPI;
        float acc[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = 0.f;
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) {
          const int g = kl + gi * LPR;
          uint32_t sdb;
          if constexpr (SLDS) sdb = SS::get(slot, 0, r * RPI + rl, g < G ? g : 0, G);
          else sdb = bt.sd[r][gi];
          const float fsd = F::scale(sdb);
          const bool live = g < G;
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            if (t < nt) {
              float dd;
              if constexpr (FMT == kFmtMxfp4)
                dd = fsd * dot_group_mx(bt.d[r][gi], xa[t][gi]);
              else
                dd = fsd * (dot_group_f16(bt.d[r][gi], xa[t][gi]) - corr[t][gi]);
              acc[t] += live ? dd : 0.f;
            }
          }
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
    // Batches i0, i0 + RB, ... (nit a multiple of RB): the loop body's
    // loads are all in range, the last one or two batches are peeled, so
    // no load sits behind a branch and each reduction waits only for its
    // own batch while the next one is in flight.
    int i0 = 0;
#pragma unroll 1
    for (; i0 + 2 * RB < nit; i0 += 2 * RB) {
      load(B, i0 + RB);
      compute(A, i0);
      load(A, i0 + 2 * RB);
      compute(B, i0 + RB);
    }
    if (i0 + RB < nit) {
      load(B, i0 + RB);
      compute(A, i0);
      compute(B, i0 + RB);
    } else {
      compute(A, i0);
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

// Rows per load batch (two batches are in flight per wave).
constexpr int rb_for(int gpl) { return gpl == 1 ? 4 : gpl == 2 ? 2 : 1; }

// Row iterations per wave: the launch is spread over about MOE_GEMV_WAVES
// waves per token held in registers (more tokens, more VALU per byte, more
// waves), every wave streaming a multiple of its batch.
int rows_per_wave(int N, int rpi, int buckets, int rb, int mt, int waves_per_token = MOE_GEMV_WAVES) {
  const int64_t row_iters = (int64_t)((N + rpi - 1) / rpi) * buckets;
  const int64_t waves = (int64_t)waves_per_token * mt;
  int64_t nit = (row_iters + waves - 1) / waves;
  nit = (nit + rb - 1) / rb * rb;
  if (nit < rb) nit = rb;
  if (nit > 64) nit = 64;
  return (int)nit;
}

#define MOE_GEMV_CASES(X) \
  X(4, 1) X(8, 1) X(16, 1) X(32, 1) X(64, 1) X(64, 2) X(64, 3) X(64, 4)

// Scales of a batch go through LDS when their chunk starts are 16-byte
// aligned (K/32 scales of SB bytes per row, a multiple of 16 bytes).
template <int FMT>
bool scales_via_lds(int K) {
  return (K / 32) * (int)sizeof(typename GemvFmt<FMT>::S) % 16 == 0;
}

template <int FMT>
hipError_t gemv_gate_up_launch(const Buckets& b, int max_buckets, const uint16_t* x, int H,
                               int I, const uint8_t* gq, const void* gs, const uint8_t* uq,
                               const void* us, uint16_t* h, float* y_zero, int64_t y_elems,
                               const Launch& L, const RouteArgs* route) {  const GemvShape sh = pick_shape(H);
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
  const int nit = rows_per_wave(I, 64 / sh.lpr, buckets, rb_for(sh.gpl), mt);
  const int rpb = kGuWaves * nit * (64 / sh.lpr);
  const bool slds = scales_via_lds<FMT>(H);
  dim3 grid((I + rpb - 1) / rpb, buckets);
#define GU(LP, GP, MTv, RV)                                                                      \
  do {                                                                                           \
    if (slds)                                                                                    \
      MOE_LAUNCH(L, (gemv_gate_up_kernel<LP, GP, MTv, rb_for(GP), RV, true, FMT>), grid,         \
                 dim3(64 * kGuWaves), 0, b, x, H, I, gq, gs, uq, us, h, y_zero, y_elems, nit, ra);         \
    else                                                                                         \
      MOE_LAUNCH(L, (gemv_gate_up_kernel<LP, GP, MTv, rb_for(GP), RV, false, FMT>), grid,        \
                 dim3(64 * kGuWaves), 0, b, x, H, I, gq, gs, uq, us, h, y_zero, y_elems, nit, ra);         \
  } while (0)
#define X(LP, GP)                                                                                \
  if (sh.lpr == LP && sh.gpl == GP) {                                                            \
    if (rv > 0) {                                                                                \
      switch (rv * 8 + mt) {                                                                     \
        case 9: GU(LP, GP, 1, 1); break;                                                         \
        case 10: GU(LP, GP, 2, 1); break;                                                        \
        case 17: GU(LP, GP, 1, 2); break;                                                        \
        case 18: GU(LP, GP, 2, 2); break;                                                        \
        case 25: GU(LP, GP, 1, 3); break;                                                        \
        case 26: GU(LP, GP, 2, 3); break;                                                        \
        case 33: GU(LP, GP, 1, 4); break;                                                        \
        case 34: GU(LP, GP, 2, 4); break;                                                        \
        default: if (GP == 1 && mt == 4) GU(LP, 1, 4, 4); else return hipErrorInvalidValue;     \
      }                                                                                          \
    } else {                                                                                     \
      switch (mt) {                                                                              \
        case 1: GU(LP, GP, 1, 0); break;                                                         \
        case 2: GU(LP, GP, 2, 0); break;                                                         \
        default: if (GP == 1) GU(LP, 1, 4, 0); break;                                            \
      }                                                                                          \
    }                                                                                            \
    return hipGetLastError();                                                                    \
  }
  MOE_GEMV_CASES(X)
#undef X
#undef GU
  return hipErrorInvalidValue;
}

template <int FMT>
hipError_t gemv_down_launch(const Buckets& b, int max_buckets, const uint16_t* h, int H, int I,
                            const uint8_t* dq, const void* ds, const float* w,
                            const float* gate_logit, int gate_ld, float* y, const Launch& L) {
  const GemvShape sh = pick_shape(I);
  const int mt = pow2_floor_min(b.max_rows, sh.gpl == 1 ? 4 : sh.gpl == 2 ? 2 : 1);
  const int buckets = b.shared_T > 0 ? 1 : max_buckets;
  // down rows are short (K = I): with one token per pass, shorter waves keep
  // more rows in flight
  const int nit = rows_per_wave(H, 64 / sh.lpr, buckets, rb_for(sh.gpl), mt,
                                mt == 1 ? MOE_GEMV_WAVES_DOWN1 : MOE_GEMV_WAVES);
  const int rpb = kDnWaves * nit * (64 / sh.lpr);
  const bool slds = scales_via_lds<FMT>(I);
  dim3 grid((H + rpb - 1) / rpb, buckets);
#define DN(LP, GP, MTv)                                                                          \
  do {                                                                                           \
    if (slds)                                                                                    \
      MOE_LAUNCH(L, (gemv_down_kernel<LP, GP, MTv, rb_for(GP), true, FMT>), grid, dim3(64 * kDnWaves), 0,  \
                 b, h, H, I, dq, ds, w, gate_logit, gate_ld, y, nit);                            \
    else                                                                                         \
      MOE_LAUNCH(L, (gemv_down_kernel<LP, GP, MTv, rb_for(GP), false, FMT>), grid, dim3(64 * kDnWaves), 0, \
                 b, h, H, I, dq, ds, w, gate_logit, gate_ld, y, nit);                            \
  } while (0)
#define X(LP, GP)                                                                                \
  if (sh.lpr == LP && sh.gpl == GP) {                                                            \
    switch (mt) {                                                                                \
      case 1: DN(LP, GP, 1); break;                                                              \
      case 2: if (GP <= 2) DN(LP, (GP <= 2 ? GP : 1), 2); break;                                 \
      default: if (GP == 1) DN(LP, 1, 4); break;                                                 \
    }                                                                                            \
    return hipGetLastError();                                                                    \
  }
  MOE_GEMV_CASES(X)
#undef X
#undef DN
  return hipErrorInvalidValue;
}

}  // namespace

// The MXFP4 instantiations (gemv_mxfp4.hip).
hipError_t launch_gemv_gate_up_mxfp4(const Buckets& b, int max_buckets, const uint16_t* x, int H,
                                     int I, const uint8_t* gq, const void* gs, const uint8_t* uq,
                                     const void* us, uint16_t* h, float* y_zero, int64_t y_elems,
                                     const Launch& L, const RouteArgs* route);
hipError_t launch_gemv_down_mxfp4(const Buckets& b, int max_buckets, const uint16_t* h, int H,
                                  int I, const uint8_t* dq, const void* ds, const float* w,
                                  const float* gate_logit, int gate_ld, float* y, const Launch& L);

}  // namespace moe
