// Routing: router logits GEMM (fp32 MFMA), softmax -> top-k -> renormalise
// (one wave64 per token), token-to-expert permutation and the expert
// schedule, and a fused single-workgroup route kernel for small batches.
//
// Sources: the dasLLAMA vulkan PR #3988 routed-block commits (router GEMM over
// the normed rows and the f32 router plane, with a gated shared expert's gate
// row after the expert rows; per-row top-k with position-major picks and
// weights; the bucket schedule in one workgroup - a count per expert,
// exclusive scans placing the buckets and the tiles, the slot map in slot
// order, an upper-bound dispatch whose unused tail is marked so that surplus
// workgroups return at once - and its later atomic tally over workgroup
// memory) and the vllm.cpp PR #481 warp router (one warp per token with the
// whole logit row in registers, a single read of the row, no shared memory,
// k rounds of arg-max then mask).
#include "device.h"
#include "kernels.h"
#include "topk.h"

#include <type_traits>

namespace moe {

// ---------------------------------------------------------------------------
// Logits L[t][e] = sum_h x[t][h] * Wr[e][h], plus column E = x[t] . g when a
// gate row is given.  One workgroup computes a 16-token x 16-row tile with
// v_mfma_f32_16x16x4_f32.  Its 16 waves each own one contiguous sixteenth of
// H (in 16-wide chunks) and issue the loads of 8 chunks before their MFMAs,
// so a wave waits about one memory latency per 8 chunks; the 16 partial tiles
// are added through LDS.  Within a chunk lane (i, q) = (lane % 16, lane / 16)
// feeds A[i][q] = x[t0+i][c+4q+r] and B[q][i] = Wr[e0+i][c+4q+r] to the r-th
// of four MFMAs, so the four MFMAs together contract the 16 inputs c..c+15
// (each lane reads 4 consecutive inputs with one vector load).
// ---------------------------------------------------------------------------
constexpr int kLogitWaves = 16;
constexpr int kLogitBatch = 8;  // chunks whose loads are in flight together

__global__ __launch_bounds__(64 * kLogitWaves) void router_logits_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr,
    const float* __restrict__ gate_row, int T, int H, int E, float* out, int ld,
    uint16_t* __restrict__ x16) {
  // The first column of tiles also writes the MFMA path's fp16 copy of its
  // 16 token rows (it reads them anyway).
  if (x16 && blockIdx.y == 0) {
    const int t0 = blockIdx.x * 16, nt = min(16, T - t0);
    const int64_t chunks = (int64_t)nt * H / 8;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + (int64_t)t0 * H);
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(x16 + (int64_t)t0 * H);
    for (int64_t c = threadIdx.x; c < chunks; c += blockDim.x) dst[c] = bf16x8_to_f16_perm8(src[c]);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, q = lane >> 4;
  const int t = blockIdx.x * 16 + i;
  const int e = blockIdx.y * 16 + i;
  const uint16_t* xrow = (t < T) ? x + (int64_t)t * H : nullptr;
  const float* wrow = nullptr;
  if (e < E) wrow = wr + (int64_t)e * H;
  else if (e == E && gate_row) wrow = gate_row;

  const int nch = H / 16;
  const int c0 = (int)((int64_t)nch * wave / kLogitWaves);
  const int c1 = (int)((int64_t)nch * (wave + 1) / kLogitWaves);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int cb = c0; cb < c1; cb += kLogitBatch) {
    uint2 xv[kLogitBatch];
    float4 wv[kLogitBatch];
#pragma unroll
    for (int u = 0; u < kLogitBatch; ++u) {
      const int kk = 16 * min(cb + u, c1 - 1) + 4 * q;
      xv[u] = xrow ? *reinterpret_cast<const uint2*>(xrow + kk) : make_uint2(0, 0);
      wv[u] = wrow ? *reinterpret_cast<const float4*>(wrow + kk) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kLogitBatch; ++u) {
      if (cb + u < c1) {
        const float a[4] = {__uint_as_float(xv[u].x << 16), __uint_as_float(xv[u].x & 0xFFFF0000u),
                            __uint_as_float(xv[u].y << 16), __uint_as_float(xv[u].y & 0xFFFF0000u)};
        const float bb[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], bb[r], acc, 0, 0, 0);
      }
    }
  }

  __shared__ f32x4_t part[kLogitWaves][64];
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4_t sum = part[0][lane];
#pragma unroll
    for (int w = 1; w < kLogitWaves; ++w) sum += part[w][lane];
    // D[4*(lane/16) + r][lane % 16]: row = token, column = router row.
    const int col = blockIdx.y * 16 + i;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = blockIdx.x * 16 + 4 * q + r;
      if (row < T && col < ld) out[(int64_t)row * ld + col] = sum[r];
    }
  }
}

hipError_t launch_router_logits(const uint16_t* x, const float* wr, const float* gate_row, int T,
                                int H, int E, float* out, int ld, uint16_t* x16, const Launch& L) {
  dim3 grid((T + 15) / 16, (ld + 15) / 16);
  MOE_LAUNCH(L, router_logits_kernel, grid, dim3(64 * kLogitWaves), 0, x, wr, gate_row, T, H, E,
             out, ld, x16);
  return hipGetLastError();
}

// Four waves per workgroup, 64/G tokens per wave.
template <int V, int G>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int ld,
                                                   int T, int E, int k, RouterSpec rs,
                                                   int32_t* __restrict__ idx,
                                                   float* __restrict__ w) {
  const int t0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / G);
  if (t0 >= T) return;
  topk_group<V, G>(logits, ld, T, t0, E, k, rs, idx, w);
}

// Calls f(integral_constant V, integral_constant G) for the (V, G) that serves (E, k).
template <typename F>
hipError_t topk_dispatch(int E, int k, F&& f) {
  const int G = topk_group_lanes(E, k);
  const int V = (E + G - 1) / G;
  if (V < 1 || V > 4) return hipErrorInvalidValue;
#define MOE_TOPK_CASE(VV, GG) \
  if (V == VV && G == GG)       \
    return f(std::integral_constant<int, VV>{}, std::integral_constant<int, GG>{});
  MOE_TOPK_CASE(1, 16) MOE_TOPK_CASE(2, 16) MOE_TOPK_CASE(3, 16) MOE_TOPK_CASE(4, 16)
  MOE_TOPK_CASE(1, 32) MOE_TOPK_CASE(2, 32) MOE_TOPK_CASE(3, 32) MOE_TOPK_CASE(4, 32)
  MOE_TOPK_CASE(1, 64) MOE_TOPK_CASE(2, 64) MOE_TOPK_CASE(3, 64) MOE_TOPK_CASE(4, 64)
#undef MOE_TOPK_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_topk(const float* logits, int ld, int T, int E, int k, const RouterSpec& rs,
                       int32_t* idx, float* w, const Launch& L) {
  return topk_dispatch(E, k, [&](auto vc, auto gc) {
    constexpr int V = decltype(vc)::value, G = decltype(gc)::value;
    const int per_block = 4 * (64 / G);
    MOE_LAUNCH(L, (topk_kernel<V, G>), dim3((T + per_block - 1) / per_block), dim3(256), 0,
               logits, ld, T, E, k, rs, idx, w);
    return hipGetLastError();
  });
}

// ---------------------------------------------------------------------------
// Permutation.  One 1024-thread workgroup: LDS histogram with LDS atomics,
// LDS scan, then a stable scatter that ranks equal experts inside each wave
// with ballots and across the 16 waves with per-wave counts, so the
// within-bucket order is ascending slot order and the result deterministic.
// ---------------------------------------------------------------------------
namespace {

constexpr int kMaxE = 256;
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// Exclusive scan of v over the workgroup's first 256 threads (the others must
// pass 0, so only the first four waves' totals can be non-zero; their results
// are meaningless).  Every thread of the workgroup (256 or more threads) must
// call it.  tmp: >= 4 ints.
__device__ int scan256(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o, 64);
    if (lane >= o) inc += n;
  }
  if (lane == 63 && wave < 4) tmp[wave] = inc;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {  // four independent LDS reads
    const int tw = tmp[w];
    pre += w < wave ? tw : 0;
    tot += tw;
  }
  *total = tot;
  __syncthreads();
  return pre + inc - v;
}

// Schedule words from the per-expert counts and offsets held in LDS.
// Touched experts in ascending order.  MFMA tiles: first every tile of the
// experts with more than 32 rows, in expert order (an expert's tiles stay
// adjacent, so they run together and share its weights in L2), then the
// one-tile experts of at most 32 rows, which fill the launch's tail.
// At most max_tiles tiles are written (the schedule buffer's capacity).
__device__ void write_schedule(const int* cnt, const int* offs, int E, int max_tiles,
                               int32_t* sched, int* tmp) {
  const int e = threadIdx.x;
  const int c = (e < E) ? cnt[e] : 0;
  const int touched = c > 0 ? 1 : 0;
  const int ntile = (c + kGemmTileRows - 1) / kGemmTileRows;
  const bool thin = touched && c <= 32;
  int n_touched, n_wide, n_thin;
  const int tpos = scan256(touched, tmp, &n_touched);
  const int wpos = scan256(thin ? 0 : ntile, tmp, &n_wide);
  const int npos = scan256(thin ? 1 : 0, tmp, &n_thin);
  const int tilepos = thin ? n_wide + npos : wpos;
  if (e < E) {
    if (touched)
      reinterpret_cast<int4*>(sched + sched_touched_offset())[tpos] = make_int4(e, offs[e], c, 0);
    int4* tiles = reinterpret_cast<int4*>(sched + sched_tiles_offset(E));
    for (int j = 0; j < ntile && tilepos + j < max_tiles; ++j) {
      const int rows = min(kGemmTileRows, c - j * kGemmTileRows);
      tiles[tilepos + j] = make_int4(e, offs[e] + j * kGemmTileRows, rows, 0);
    }
  }
  if (threadIdx.x == 0) {
    sched[0] = n_touched;
    sched[1] = min(n_wide + n_thin, max_tiles);
    sched[2] = n_thin;  // the list's last n_thin tiles are the one-tile thin experts'
  }
}

}  // namespace

struct PermuteLds {
  int cnt[kMaxE];
  int offs[kMaxE];
  int cursor[kMaxE];
  int wcnt[kWaves][kMaxE];
  int tmp[kWaves];
};

// idx may point to global or LDS memory.  Every thread of the workgroup calls.
__device__ void permute_block(const int32_t* idx, int S, int E, int32_t* __restrict__ off,
                              int32_t* __restrict__ sorted, int32_t* __restrict__ row_of,
                              int32_t* __restrict__ sched, int max_tiles, PermuteLds& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int i = tid; i < kMaxE; i += kThreads) sm.cnt[i] = 0;
  __syncthreads();
  for (int s = tid; s < S; s += kThreads) {
    const int e = idx[s];
    if (e >= 0 && e < E) atomicAdd(&sm.cnt[e], 1);
  }
  __syncthreads();

  int total;
  const int pre = scan256((tid < E) ? sm.cnt[tid] : 0, sm.tmp, &total);
  if (tid < E) {
    sm.offs[tid] = pre;
    sm.cursor[tid] = pre;
    off[tid] = pre;
  }
  if (tid == 0) off[E] = total;
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < S; base += kThreads) {
    const int s = base + tid;
    int e = (s < S) ? idx[s] : -1;
    if (e >= E) e = -1;
    for (int i = tid; i < kWaves * kMaxE; i += kThreads) (&sm.wcnt[0][0])[i] = 0;
    __syncthreads();
    // Lanes of this wave holding the same expert (key e + 1 fits in 9 bits).
    const int key = e + 1;
    uint64_t peers = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 9; ++bit) {
      const uint64_t bal = __ballot((key >> bit) & 1);
      peers &= ((key >> bit) & 1) ? bal : ~bal;
    }
    const int rank = __popcll(peers & lt_mask);
    if (e >= 0 && rank == 0) sm.wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (e >= 0) {
      int pos = sm.cursor[e] + rank;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) pos += w < wave ? sm.wcnt[w][e] : 0;
      sorted[pos] = s;
      row_of[s] = pos;
    } else if (s < S) {
      row_of[s] = -1;
    }
    __syncthreads();
    if (tid < E) {
      int add = 0;
      for (int w = 0; w < kWaves; ++w) add += sm.wcnt[w][tid];
      sm.cursor[tid] += add;
    }
    __syncthreads();
  }

  if (sched) write_schedule(sm.cnt, sm.offs, E, max_tiles, sched, sm.tmp);
}

__global__ __launch_bounds__(kThreads) void permute_kernel(const int32_t* __restrict__ idx, int S,
                                                           int E, int32_t* __restrict__ off,
                                                           int32_t* __restrict__ sorted,
                                                           int32_t* __restrict__ row_of,
                                                           int32_t* __restrict__ sched,
                                                           int max_tiles) {
  __shared__ PermuteLds sm;
  permute_block(idx, S, E, off, sorted, row_of, sched, max_tiles, sm);
}

// Fused routing for small batches: the workgroup's 16 waves run the top-k of
// every token (64/G tokens per wave at a time), keep the picks in LDS, and the
// same workgroup then builds the permutation and schedule from them.
template <int V, int G>
__global__ __launch_bounds__(kThreads) void route_kernel(const float* __restrict__ logits, int ld,
                                                         int T, int E, int k, RouterSpec rs,
                                                         int32_t* __restrict__ idx,
                                                         float* __restrict__ w,
                                                         int32_t* __restrict__ off,
                                                         int32_t* __restrict__ sorted,
                                                         int32_t* __restrict__ row_of,
                                                         int32_t* __restrict__ sched,
                                                         int max_tiles) {
  __shared__ PermuteLds sm;
  __shared__ int32_t picks[kRouteMaxSlots];
  constexpr int TPW = 64 / G;
  for (int t0 = (threadIdx.x >> 6) * TPW; t0 < T; t0 += kWaves * TPW)
    topk_group<V, G>(logits, ld, T, t0, E, k, rs, idx, w, picks, nullptr, 0);
  __syncthreads();
  permute_block(picks, T * k, E, off, sorted, row_of, sched, max_tiles, sm);
}

hipError_t launch_route(const float* logits, int ld, int T, int E, int k, const RouterSpec& rs,
                        int32_t* idx, float* w, int32_t* off, int32_t* sorted,
                        int32_t* row_of, int32_t* sched, const Launch& L) {
  const int max_tiles = (int)sched_max_tiles((int64_t)T * k, E);
  return topk_dispatch(E, k, [&](auto vc, auto gc) {
    constexpr int V = decltype(vc)::value, G = decltype(gc)::value;
    MOE_LAUNCH(L, (route_kernel<V, G>), dim3(1), dim3(kThreads), 0, logits, ld, T, E, k,
               rs, idx, w, off, sorted, row_of, sched, max_tiles);
    return hipGetLastError();
  });
}

// The schedule alone, from offsets written earlier (for callers that bring
// their own permutation).  One 256-thread workgroup.
__global__ __launch_bounds__(256) void schedule_kernel(const int32_t* __restrict__ off, int E,
                                                       int32_t* __restrict__ sched,
                                                       int max_tiles) {
  __shared__ int cnt[kMaxE];
  __shared__ int offs[kMaxE];
  __shared__ int tmp[4];
  const int e = threadIdx.x;
  if (e < E) {
    offs[e] = off[e];
    cnt[e] = off[e + 1] - off[e];
  }
  __syncthreads();
  write_schedule(cnt, offs, E, max_tiles, sched, tmp);
}

// ---------------------------------------------------------------------------
// Permutation over many workgroups (large slot counts).  Slots are cut into
// blocks of kThreads; (1) each block counts its slots per expert, (2) one
// workgroup turns the counts into bucket offsets, each block's first position
// inside every bucket, and the tile schedule, (3) each block scatters its
// slots, ranking equal experts in slot order exactly as the one-workgroup
// version does, so the result is the same stable permutation.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void block_count_kernel(const int32_t* __restrict__ idx,
                                                               int S, int E,
                                                               int32_t* __restrict__ bcnt) {
  __shared__ int cnt[kMaxE];
  for (int i = threadIdx.x; i < kMaxE; i += kThreads) cnt[i] = 0;
  __syncthreads();
  const int s = blockIdx.x * kThreads + threadIdx.x;
  if (s < S) {
    const int e = idx[s];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) bcnt[(int64_t)blockIdx.x * E + e] = cnt[e];
}

__global__ __launch_bounds__(256) void block_offsets_kernel(int32_t* __restrict__ bcnt, int nblk,
                                                            int E, int32_t* __restrict__ off,
                                                            int32_t* __restrict__ sched,
                                                            int max_tiles) {
  __shared__ int cnt[kMaxE];
  __shared__ int offs[kMaxE];
  __shared__ int tmp[4];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E)
    for (int b0 = 0; b0 < nblk; b0 += 8) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = (b0 + u < nblk) ? bcnt[(int64_t)(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (b0 + u < nblk) {
          bcnt[(int64_t)(b0 + u) * E + e] = run;  // block's position inside bucket e
          run += c[u];
        }
    }
  int total;
  const int pre = scan256(e < E ? run : 0, tmp, &total);
  if (e < E) {
    cnt[e] = run;
    offs[e] = pre;
    off[e] = pre;
  }
  if (e == 0) off[E] = total;
  __syncthreads();
  if (sched) write_schedule(cnt, offs, E, max_tiles, sched, tmp);
}

__global__ __launch_bounds__(kThreads) void block_scatter_kernel(const int32_t* __restrict__ idx,
                                                                 int S, int E,
                                                                 const int32_t* __restrict__ bpos,
                                                                 const int32_t* __restrict__ off,
                                                                 int32_t* __restrict__ sorted,
                                                                 int32_t* __restrict__ row_of) {
  __shared__ int wcnt[kWaves][kMaxE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = blockIdx.x * kThreads + tid;
  int e = (s < S) ? idx[s] : -1;
  if (e >= E) e = -1;
  for (int i = tid; i < kWaves * kMaxE; i += kThreads) (&wcnt[0][0])[i] = 0;
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int key = e + 1;
  uint64_t peers = ~0ull;
#pragma unroll
  for (int bit = 0; bit < 9; ++bit) {
    const uint64_t bal = __ballot((key >> bit) & 1);
    peers &= ((key >> bit) & 1) ? bal : ~bal;
  }
  const int rank = __popcll(peers & lt_mask);
  if (e >= 0 && rank == 0) wcnt[wave][e] = __popcll(peers);
  __syncthreads();
  if (e >= 0) {
    int pos = off[e] + bpos[(int64_t)blockIdx.x * E + e] + rank;
    for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
    sorted[pos] = s;
    row_of[s] = pos;
  } else if (s < S) {
    row_of[s] = -1;
  }
}

hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* off,
                          int32_t* sorted, int32_t* row_of, int32_t* sched, int32_t* scratch,
                          const Launch& L) {
  const int S = T * k;
  const int max_tiles = (int)sched_max_tiles((int64_t)S, E);
  if (!scratch || S <= kPermuteOneBlockMax) {
    MOE_LAUNCH(L, permute_kernel, dim3(1), dim3(kThreads), 0, idx, S, E, off, sorted, row_of,
               sched, max_tiles);
    return hipGetLastError();
  }
  // the first launch carries the caller's start event, the last its stop
  const int nblk = (S + kThreads - 1) / kThreads;
  const Launch first{L.st, L.start, nullptr}, mid{L.st, nullptr, nullptr}, last{L.st, nullptr, L.stop};
  MOE_LAUNCH(first, block_count_kernel, dim3(nblk), dim3(kThreads), 0, idx, S, E, scratch);
  MOE_LAUNCH(mid, block_offsets_kernel, dim3(1), dim3(256), 0, scratch, nblk, E, off, sched,
             max_tiles);
  MOE_LAUNCH(last, block_scatter_kernel, dim3(nblk), dim3(kThreads), 0, idx, S, E, scratch, off,
             sorted, row_of);
  return hipGetLastError();
}

hipError_t launch_schedule_from_offsets(const int32_t* off, int E, int64_t slots, int32_t* sched,
                                        const Launch& L) {
  MOE_LAUNCH(L, schedule_kernel, dim3(1), dim3(256), 0, off, E, sched,
                     (int)sched_max_tiles(slots, E));
  return hipGetLastError();
}

}  // namespace moe
