// Host-side launchers of the libmoe kernels.  Every launcher enqueues on the
// given stream and returns the launch status; argument checking happens in
// moe_api.cpp before any of these is called.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Where a kernel is enqueued.  With start/stop events set, the launch goes
// through hipExtLaunchKernelGGL, which records them at the kernel's own start
// and end on the stream (per-kernel device time without extra packets).
struct Launch {
  hipStream_t st;
  hipEvent_t start = nullptr, stop = nullptr;
};

#define MOE_LAUNCH(L, kernel, grid, block, shmem, ...)                                    \
  do {                                                                                    \
    if ((L).start || (L).stop)                                                            \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, (L).st, (L).start, (L).stop, 0,   \
                            __VA_ARGS__);                                                 \
    else                                                                                  \
      hipLaunchKernelGGL(kernel, grid, block, shmem, (L).st, __VA_ARGS__);                \
  } while (0)

// Schedule words written by the permutation kernels, read by the expert MLPs:
//   [0] number of experts with at least one slot (touched experts)
//   [1] number of MFMA row tiles
//   [2] how many of them, at the end of the list, belong to the one-tile
//       experts of at most 32 rows (the list's other tiles are in expert order)
//   [4 .. 4+4E)            touched experts, ascending: {expert, first row, rows, 0}
//   [tiles_offset(E) ..)   tiles, 4 ints each: {expert, first row, rows, 0}
// An expert's rows are cut into tiles of kGemmTileRows; only its last tile can
// be short.
constexpr int kGemmTileRows = 128;  // rows (slots) per MFMA tile
__host__ __device__ constexpr int sched_touched_offset() { return 4; }
__host__ __device__ constexpr int sched_tiles_offset(int E) { return 4 + 4 * E; }
__host__ __device__ constexpr int64_t sched_max_tiles(int64_t slots, int E) {
  return (slots + kGemmTileRows - 1) / kGemmTileRows + E;
}
__host__ __device__ constexpr int64_t sched_words(int64_t slots, int E) {
  return sched_tiles_offset(E) + 4 * sched_max_tiles(slots, E);
}

// Bucket description shared by the expert-MLP kernels.  Routed buckets come
// from the permutation (off, sorted, sched); the shared expert is one bucket
// over every token with the identity map (shared_T > 0).
struct Buckets {
  const int32_t* off;     // [E+1]
  const int32_t* sorted;  // [slots]
  const int32_t* sched;   // schedule words (see above)
  int32_t k;              // picks per token (slot s belongs to token s / k)
  int32_t shared_T;       // > 0: identity bucket over shared_T tokens
  int32_t max_rows;       // upper bound of rows in one bucket (T: a token picks an expert once)
  int32_t E;              // experts (locates the tile list in sched)
};

// x16 (nullable): also write the fp16 operand-order copy of x (as
// launch_convert_x16 does).
hipError_t launch_router_logits(const uint16_t* x, const float* wr, const float* gate_row, int T,
                                int H, int E, float* out, int ld, uint16_t* x16, const Launch& L);

// How a token's picks and weights are formed.
//   route_scale : multiplies the renormalised weights.
//   top_p       : expert top-p after the top-k (0 < top_p < 1; other values
//                 keep all k); a dropped pick is written as index -1, weight 0.
//                 Plain softmax router only.
//   score, bias : router variant.  score 0 = softmax probability, 1 = sigmoid
//                 of the logit; bias (nullable, fp32 [E]) is added to the
//                 score for the selection only.  With score 0, no bias and no
//                 grouping the plain router runs (selection on the logits
//                 themselves).
//   n_group, topk_group : grouped routing when n_group > 1 (n_group divides
//                 E, at most kMaxGroups; 1 <= topk_group <= n_group): only
//                 the experts of the topk_group groups with the largest
//                 top-2 key sums can be picked.
constexpr int kMaxGroups = 16;
struct RouterSpec {
  float route_scale;
  float top_p;
  int score;
  const float* bias;
  int n_group = 0;
  int topk_group = 0;
  __host__ __device__ bool variant() const {
    return score != 0 || bias != nullptr || n_group > 1;
  }
};

hipError_t launch_topk(const float* logits, int ld, int T, int E, int k, const RouterSpec& rs,
                       int32_t* idx, float* w, const Launch& L);

// Fused top-k + permutation in one workgroup, for up to kRouteMaxSlots slots
// and kRouteMaxT tokens (4 tokens per wave of the 16).
constexpr int kRouteMaxSlots = 4096;
constexpr int kRouteMaxT = 64;
hipError_t launch_route(const float* logits, int ld, int T, int E, int k, const RouterSpec& rs,
                        int32_t* idx, float* w, int32_t* off, int32_t* sorted,
                        int32_t* row_of, int32_t* sched, const Launch& L);

// Stable permutation (+ schedule when sched is given).  Up to
// kPermuteOneBlockMax slots, or without scratch, one workgroup does it all;
// beyond, three launches over blocks of 1024 slots use scratch
// (permute_scratch_words ints).
constexpr int kPermuteOneBlockMax = 4096;
__host__ __device__ constexpr int64_t permute_scratch_words(int64_t slots, int E) {
  return ((slots + 1023) / 1024) * E;
}
hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* off,
                          int32_t* sorted, int32_t* row_of, int32_t* sched, int32_t* scratch,
                          const Launch& L);

hipError_t launch_schedule_from_offsets(const int32_t* off, int E, int64_t slots, int32_t* sched,
                                        const Launch& L);

// Routing folded into the gate/up GEMV for very small batches (T <=
// kFusedRouteMaxT tokens, T*k <= kFusedRouteMaxSlots slots): every workgroup
// redoes the (deterministic) top-k and bucket build in registers, and
// workgroup (0,0) publishes idx, w, sorted, row_of and the schedule for the
// down launch, and off for more than one token (one token's rows follow the
// rank of the pick, not the expert order).
#ifndef MOE_FUSED_ROUTE_MAX_T
#define MOE_FUSED_ROUTE_MAX_T 4
#endif
constexpr int kFusedRouteMaxT = MOE_FUSED_ROUTE_MAX_T;
constexpr int kFusedRouteMaxSlots = 64;
struct RouteArgs {
  const float* logits;  // [T][ld]
  int ld, E, T;
  RouterSpec rs;
  int32_t* idx;     // [T][k]
  float* w;         // [T][k]
  int32_t* off;     // [E+1]
  int32_t* sorted;  // [T*k]
  int32_t* row_of;  // [T*k]
  int32_t* sched;   // schedule words
};

// Weight formats: the scale pointers hold fp16 bits (kFmtInt4) or ue8m0
// bytes (kFmtMxfp4).
enum WeightFormat : int { kFmtInt4 = 0, kFmtMxfp4 = 1 };

// Streaming 4-bit GEMV (decode).  gate/up: h[row][I] = fp16(silu(Wg x)*(Wu x));
// down: y[token] += weight * (Wd h[row]).  The gate/up launch also zeroes y.
hipError_t launch_gemv_gate_up(const Buckets& b, int max_buckets, const uint16_t* x, int H,
                               int I, const uint8_t* gq, const void* gs, const uint8_t* uq,
                               const void* us, uint16_t* h, float* y_zero, int64_t y_elems,
                               int fmt, const Launch& L, const RouteArgs* route = nullptr);
hipError_t launch_gemv_down(const Buckets& b, int max_buckets, const uint16_t* h, int H, int I,
                            const uint8_t* dq, const void* ds, const float* w,
                            const float* gate_logit, int gate_ld, float* y, int fmt,
                            const Launch& L);
bool gemv_supported(int K);

// The same two GEMVs over tiled planes (gemv_tiled.hip): a workgroup per
// 32-row block row of a bucket, its four waves splitting K.  Bucket and
// routing arguments as above.
hipError_t launch_gemv_tiled_gate_up(const Buckets& b, int max_buckets, const uint16_t* x, int H,
                                     int I, const uint8_t* gq, const void* gs, const uint8_t* uq,
                                     const void* us, uint16_t* h, float* y_zero, int64_t y_elems,
                                     int fmt, const Launch& L, const RouteArgs* route = nullptr);
hipError_t launch_gemv_tiled_down(const Buckets& b, int max_buckets, const uint16_t* h, int H,
                                  int I, const uint8_t* dq, const void* ds, const float* w,
                                  const float* gate_logit, int gate_ld, float* y, int fmt,
                                  const Launch& L);
bool gemv_tiled_supported(int K);

// Grouped MFMA GEMM (prefill), fp16 operands with fp32 accumulation.
// Row layout -> tiled layout of E experts' planes q [E][N][K/2], s [E][N][K/32]
// (scale elements of the format fmt).
hipError_t launch_pack_weights(const uint8_t* sq, const void* ss, int E, int N, int K,
                               uint8_t* dq, void* ds, int fmt, const Launch& L);

// n[t] = bf16(r[t] * g / sqrt(mean(r[t]^2) + eps)) for T rows of H (H % 4 == 0).
hipError_t launch_rmsnorm(const float* r, const float* g, int T, int H, float eps, uint16_t* out,
                          const Launch& L);

// The same, plus the next layer's router logits of the normed bf16 rows,
// logits[t][e] = sum_h n[t][h] * wr[e][h] (fp32 [T][E]).  One launch (the
// router folded into the norm kernel) when fold_router_served(T, H); else
// the norm launch and then the router-logits kernel over n.
constexpr int kFoldRouterRows = 4;     // token rows per workgroup of the fold
constexpr int kFoldRouterMaxT = 32;    // larger batches take the two launches
constexpr int kFoldRouterMaxH = 6144;  // the normed rows live in LDS (48 KiB)
__host__ __device__ constexpr bool fold_router_served(int T, int H) {
  return T <= kFoldRouterMaxT && H <= kFoldRouterMaxH;
}
hipError_t launch_rmsnorm_router(const float* r, const float* g, int T, int H, float eps,
                                 uint16_t* out, const float* wr, int E, float* logits,
                                 const Launch& L);

// bf16 x [T][H] -> fp16 copy with each block of 8 in the order 0,4,1,5,2,6,3,7.
hipError_t launch_convert_x16(const uint16_t* x, int T, int H, uint16_t* x16, const Launch& L);

// The shared expert as extra tiles of the grouped-GEMM launches: identity
// rows over all T tokens, planes gate/up/down, hidden rows h16 [T][SI], and
// the down pass weighting row t by sigmoid(gate_logit[t * gate_ld]) (1 when
// gate_logit is null).
struct SharedGemm {
  int T, SI;
  const uint8_t* q[3];
  const void* s[3];  // scales in the call's weight format
  uint16_t* h16;
  const float* gate_logit;
  int gate_ld;
};

// x16: the activations in fp16, operand order (launch_convert_x16).  The
// launch also clears y_zero[0 .. y_elems) (y_elems a multiple of 4) for the
// down pass's atomic combine.
// tiled: every plane (shared ones included) is in the tiled layout.
// fmt: the weight format of every plane (WeightFormat).
hipError_t launch_gemm_gate_up(const Buckets& b, int max_tiles, const uint16_t* x16, int H,
                               int I, const uint8_t* gq, const void* gs,
                               const uint8_t* uq, const void* us, uint16_t* h16,
                               const SharedGemm* shared, float* y_zero, int64_t y_elems,
                               bool tiled, int fmt, const Launch& L);
hipError_t launch_gemm_down(const Buckets& b, int max_tiles, const uint16_t* h16, int H, int I,
                            const uint8_t* dq, const void* ds, const float* w, float* y,
                            const SharedGemm* shared, bool tiled, int fmt, const Launch& L);

// Streaming-read probe over bytes (a multiple of 16) of src with the given
// number of 256-thread workgroups; sink holds 256 words (written only in a
// case the probe's inputs never produce).
hipError_t launch_read_probe(const void* src, int64_t bytes, int workgroups, uint32_t* sink,
                             const Launch& L);

// Decoders the debug hook runs (s holds fp16 bits for the int4 ones, ue8m0
// bytes for the MXFP4 ones).
enum DebugDecoder : int {
  kDebugQ4GemvGateUp = 0,  // q4_bf16_pairs (gate/up GEMV), exact weight
  kDebugQ4Mfma = 1,        // q4_f16x8 (MFMA tiles of 2-4 row subtiles), fp16 operand
  kDebugQ4MfmaCvt = 2,     // q4_f16x8_cvt (one-subtile MFMA tiles), fp16 operand
  kDebugQ4GemvDown = 3,    // q4_f16_pairs (down GEMV), exact weight
  kDebugMx4Gemv = 4,       // e2m1_pair x e8m0_f32 (both GEMVs), exact weight
  kDebugMx4Mfma = 5,       // mx4_f16x8 (MFMA tiles of 2-4 row subtiles), fp16 operand
  kDebugMx4MfmaCvt = 6,    // mx4_f16x8_cvt (one-subtile MFMA tiles), fp16 operand
};
hipError_t launch_debug_dequant(const uint8_t* q, const void* s, int N, int K, int mode,
                                float* out, const Launch& L);

}  // namespace moe
