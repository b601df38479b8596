// Token-to-expert permutation and the expert schedule.
//
// Source: the dasLLAMA vulkan PR #3988 bucket schedule (one workgroup; a count
// per expert, exclusive scans placing the buckets and the tiles, the slot map
// in slot order, an upper-bound dispatch whose unused tail is marked so that
// surplus workgroups return at once) and its later atomic tally over
// workgroup memory.  Here: one 1024-thread workgroup, LDS histogram with LDS
// atomics, LDS scan, then a stable scatter that ranks equal experts inside
// each wave with ballots and across the 16 waves with per-wave counts, so the
// within-bucket order is ascending slot order and the result is
// deterministic.
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kMaxE = 256;
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// Exclusive scan of v over the workgroup's first 256 threads (the others must
// pass 0).  Every thread of the workgroup must call it.  tmp: >= kWaves ints.
__device__ int scan256(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o, 64);
    if (lane >= o) inc += n;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  int pre = 0, tot = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    if (w < wave) pre += tmp[w];
    tot += tmp[w];
  }
  *total = tot;
  __syncthreads();
  return pre + inc - v;
}

// Schedule words from the per-expert counts and offsets held in LDS.
// At most max_tiles tiles are written (the schedule buffer's capacity).
__device__ void write_schedule(const int* cnt, const int* offs, int E, int max_tiles,
                               int32_t* sched, int* tmp) {
  const int e = threadIdx.x;
  const int c = (e < E) ? cnt[e] : 0;
  const int touched = c > 0 ? 1 : 0;
  const int ntile = (c + kGemmTileRows - 1) / kGemmTileRows;
  int n_touched, n_tiles;
  const int tpos = scan256(touched, tmp, &n_touched);
  const int tilepos = scan256(ntile, tmp, &n_tiles);
  if (e < E) {
    if (touched) sched[2 + tpos] = e;
    int4* tiles = reinterpret_cast<int4*>(sched + sched_tiles_offset(E));
    for (int j = 0; j < ntile && tilepos + j < max_tiles; ++j) {
      const int rows = min(kGemmTileRows, c - j * kGemmTileRows);
      tiles[tilepos + j] = make_int4(e, offs[e] + j * kGemmTileRows, rows, 0);
    }
  }
  if (threadIdx.x == 0) {
    sched[0] = n_touched;
    sched[1] = min(n_tiles, max_tiles);
  }
}

}  // namespace

__global__ __launch_bounds__(kThreads) void permute_kernel(const int32_t* __restrict__ idx, int S,
                                                           int E, int32_t* __restrict__ off,
                                                           int32_t* __restrict__ sorted,
                                                           int32_t* __restrict__ row_of,
                                                           int32_t* __restrict__ sched,
                                                           int max_tiles) {
  __shared__ int cnt[kMaxE];
  __shared__ int offs[kMaxE];
  __shared__ int cursor[kMaxE];
  __shared__ int wcnt[kWaves][kMaxE];
  __shared__ int tmp[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int i = tid; i < kMaxE; i += kThreads) cnt[i] = 0;
  __syncthreads();
  for (int s = tid; s < S; s += kThreads) {
    const int e = idx[s];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();

  int total;
  const int pre = scan256((tid < E) ? cnt[tid] : 0, tmp, &total);
  if (tid < E) {
    offs[tid] = pre;
    cursor[tid] = pre;
    off[tid] = pre;
  }
  if (tid == 0) off[E] = total;
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < S; base += kThreads) {
    const int s = base + tid;
    int e = (s < S) ? idx[s] : -1;
    if (e >= E) e = -1;
    for (int i = tid; i < kWaves * kMaxE; i += kThreads) (&wcnt[0][0])[i] = 0;
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
    if (e >= 0 && rank == 0) wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (e >= 0) {
      int pos = cursor[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
      sorted[pos] = s;
      row_of[s] = pos;
    } else if (s < S) {
      row_of[s] = -1;
    }
    __syncthreads();
    if (tid < E) {
      int add = 0;
      for (int w = 0; w < kWaves; ++w) add += wcnt[w][tid];
      cursor[tid] += add;
    }
    __syncthreads();
  }

  if (sched) write_schedule(cnt, offs, E, max_tiles, sched, tmp);
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

hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* off,
                          int32_t* sorted, int32_t* row_of, int32_t* sched, hipStream_t st) {
  const int max_tiles = (int)sched_max_tiles((int64_t)T * k, E);
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kThreads), 0, st, idx, T * k, E, off, sorted,
                     row_of, sched, max_tiles);
  return hipGetLastError();
}

hipError_t launch_schedule_from_offsets(const int32_t* off, int E, int64_t slots, int32_t* sched,
                                        hipStream_t st) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(256), 0, st, off, E, sched,
                     (int)sched_max_tiles(slots, E));
  return hipGetLastError();
}

}  // namespace moe
