// Grouped 4-bit (int4 or MXFP4) GEMM on fp16 MFMA for prefill-sized buckets.
//
// Sources: the dasLLAMA vulkan PR #3988 routed block (bucket rows gathered
// through the slot map into expert tiles, an upper-bound dispatch whose
// surplus workgroups return at once, the act step between gate/up and down,
// the combine reading each slot's row through the map; the shared expert as
// one more region over every row with an identity map, weighted by the
// sigmoid of its gate logit) and the colibri PR #418 weight formats: int4
// (nibble - 8, one fp16 scale per 32 inputs) and, from its later fmt=7
// comment, MXFP4 (e2m1 nibbles, one ue8m0 exponent per 32 inputs).
//
// gfx950 design.  A workgroup of kWaves waves (one per SIMD; two workgroups
// share a CU) owns one row tile of up to 128 bucket rows and a block of output columns.  Waves
// split the columns, so each wave decodes its own weight fragment straight
// from a 128-bit global load into MFMA operand registers (no LDS round trip
// for weights), while the activation tile - shared by all the waves - is
// staged through LDS, double-buffered, one barrier per 64-deep K step.  The
// MFMA is v_mfma_f32_32x32x16_f16:
//   A (32 rows x 16 k)  lane l: row l%32, k 8*(l/32)..+7  (activations)
//   B (16 k x 32 cols)  lane l: col l%32, k 8*(l/32)..+7  (weights)
//   D (32 x 32, fp32)   lane l: col l%32, rows 8*(v/4) + 4*(l/32) + v%4.
// The weight operand is the exact dequantised value ((nibble-8)*scale, or
// e2m1(nibble)*2^(e-127) scaled by a per-row power of two that the epilogue
// undoes, see e8m0_f16_shifted) rounded once to fp16; fp16 and bf16 MFMA
// have the same peak on gfx950, and fp16's 11-bit significand keeps the
// layer within its tolerance where bf16 would not.  Activations are fp16 copies stored with each block of 8 in the order
// 0,4,1,5,2,6,3,7, matching the nibble pairing of the decode.
//
// K mapping inside one 64-deep step: lane (j, hf) = (l%32, l/32) loads the 16
// bytes of scale group 2*step + hf of weight row j; packed word d of it feeds
// MFMA d.  MFMA d therefore contracts k = 32*hf + 8*d + {0..7}: its A operand
// is the 16 bytes at k offset 32*hf + 8*d of the LDS activation row.
//
// The down pass may split K over blockIdx.z: its epilogue already adds into
// y with atomics, so partial sums over K ranges combine the same way.
#include "device.h"
#include "kernels.h"

#ifndef MOE_GEMM_DA
#define MOE_GEMM_DA 2  // activation register stages (prefetch distance in K steps)
#endif
#ifndef MOE_GEMM_DB
#define MOE_GEMM_DB 2  // weight register stages
#endif

#ifndef MOE_GEMM_W0_AHEAD
// Decode the next K step's word 0 under this step's last MFMAs (bit 0: the
// gate/up pass, bit 1: the down pass; int4 only).  On the skewed prefill it
// takes the int4 down pass 645 -> 624 us, while gate/up and MXFP4 (whose
// conversion decode is lighter) measured equal or slower.
#define MOE_GEMM_W0_AHEAD 2
#endif

// Dispatch order of the thin experts' tiles: 0 last, 1 first, 2 spread
// evenly among the wide ones.
#ifndef MOE_GEMM_THIN_ORDER_GU
#define MOE_GEMM_THIN_ORDER_GU 0  // gate/up pass
#endif
#ifndef MOE_GEMM_THIN_ORDER_DN
#define MOE_GEMM_THIN_ORDER_DN 1  // down pass
#endif
// Rows per shared-expert tile on tiled planes (row planes keep 128): 64-row
// tiles halve the longest workgroups' MFMA chain at the cost of decoding the
// shared weights twice as often.  prefill_shared gate/up 79.5 -> 76.0 us
// (MXFP4 87.5 -> 83.7 us; 96 rows no better), down 66.2 -> 63.5 us; on row
// planes, whose weight reads are already re-fetched per K step, the down
// pass measured 79.4 -> 92.1 us.
#ifndef MOE_GEMM_SHARED_ROWS_GU
#define MOE_GEMM_SHARED_ROWS_GU 64
#endif
#ifndef MOE_GEMM_SHARED_ROWS_DN
#define MOE_GEMM_SHARED_ROWS_DN 64
#endif
#ifndef MOE_GEMM_OCC
#define MOE_GEMM_OCC 2  // workgroups per CU
#endif
#ifndef MOE_GEMM_GU_NS
#define MOE_GEMM_GU_NS 1  // 32-column subtiles per wave, gate/up pass
#endif
#ifndef MOE_GEMM_DN_NS
#define MOE_GEMM_DN_NS 2  // 32-column subtiles per wave, down pass
#endif
#ifndef MOE_GEMM_WAVES
#define MOE_GEMM_WAVES 4  // waves per workgroup (column groups)
#endif

#include <algorithm>
#include <type_traits>
#include <utility>

namespace moe {

namespace {

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), unrolled.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
constexpr int gcd_c(int x, int y) { return y == 0 ? x : gcd_c(y, x % y); }
constexpr int lcm_c(int x, int y) { return x / gcd_c(x, y) * y; }

constexpr int kBM = kGemmTileRows;    // 128 rows per tile
static_assert(MOE_GEMM_SHARED_ROWS_GU > 0 && MOE_GEMM_SHARED_ROWS_GU <= kBM &&
                  MOE_GEMM_SHARED_ROWS_GU % 32 == 0 && MOE_GEMM_SHARED_ROWS_DN > 0 &&
                  MOE_GEMM_SHARED_ROWS_DN <= kBM && MOE_GEMM_SHARED_ROWS_DN % 32 == 0,
              "shared-expert tiles hold whole 32-row subtiles, at most a tile");
constexpr int kKS = 64;               // K per step
constexpr int kPitch = kKS * 2 + 16;  // LDS row pitch in bytes (padding breaks bank conflicts)
constexpr int kWaves = MOE_GEMM_WAVES;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunkRows = kThreads / 8;  // activation rows one pass of the workgroup stages

struct TileView {
  int e, row0, nrows;
};

// Row-major fp16 position of logical column j in the permuted-by-8 layout.
__device__ __forceinline__ int perm_col(int j) { return (j & ~7) | perm8_pos(j & 7); }

// Raw weight operands of one K step for one lane: the 16 bytes of scale
// group 2*step + hf of each (subtile, plane) weight row, and its scale (fp16
// bits or a ue8m0 byte).
template <int P, int NS>
struct BStage {
  u32x4_t q[NS][P];
  uint32_t s[NS][P];
};

// Activation operands of one K step as loaded by one thread: NA 16-byte
// chunks; chunk i is row (tid/8) + kChunkRows*i, bytes 16*(tid%8) of the step.
template <int NA>
struct AStage {
  u32x4_t v[NA];
};

// One source of tiles: the routed buckets or the shared expert.
struct GemmSrc {
  const uint16_t* act;   // fp16 activations, row stride K, each block of 8 in
                         // the operand order 0,4,1,5,2,6,3,7
  int K, N;              // contraction depth and output columns of one plane
  const uint8_t* q[2];   // weight planes: [E][N][K/2] nibbles
  const void* s[2];      // and their [E][N][K/32] scales (fp16 bits or ue8m0 bytes)
  uint16_t* hout;        // MODE 0 output, row stride N
  int ksplit;            // K ranges of one tile's column block (MODE 1; 1 for MODE 0)
  int tiled;             // planes in the tiled layout (1 KB per 32 rows x 64 k)
};

struct GemmArgs {
  GemmSrc src[2];        // [0] routed buckets, [1] shared expert
  int shared_T;          // rows of the shared expert (0: none)
  int shared_tiles;      // row tiles of the shared expert
  int shared_rows;       // rows per shared-expert tile (at most kBM)
  int gx[2];             // column blocks of one tile: [0] routed, [1] shared
  const float* w;        // MODE 1 combine weights per slot
  const float* gate_logit;  // MODE 1 shared-expert gate logits (nullable)
  int gate_ld;
  float* y;              // MODE 1 output [T][H]
  int H;
  float* y_zero;         // MODE 0: output the launch clears for the down pass
  int64_t y_elems;       // (a multiple of 4)
};

// Tile, column block and K range of this workgroup.  blockIdx.x runs first
// over the shared expert's tiles (identity rows over all tokens), a.gx[1]
// column blocks times its ksplit K ranges each, then over the routed tile
// list, a.gx[0] column blocks times its ksplit each (consecutive workgroups
// share a tile, column blocks before K ranges), so each source's grid is
// exactly its own size and the long shared-expert work is dispatched first,
// all of its K ranges included.
__device__ __forceinline__ bool tile_of(const Buckets& b, const GemmArgs& a, TileView* v,
                                        int* src, int* cblk, int* kz, int order) {
  int wg = blockIdx.x;
  const int per1 = a.gx[1] * a.src[1].ksplit;
  const int shared_wgs = a.shared_tiles * per1;
  if (wg < shared_wgs) {
    const int u = wg / per1, r = wg - u * per1;
    *kz = r / a.gx[1];
    *cblk = r - *kz * a.gx[1];
    *src = 1;
    v->e = 0;
    v->row0 = u * a.shared_rows;
    v->nrows = min(a.shared_rows, a.shared_T - v->row0);
    return v->nrows > 0;
  }
  wg -= shared_wgs;
  const int per0 = a.gx[0] * a.src[0].ksplit;
  int u = wg / per0;
  const int r = wg - u * per0;
  *kz = r / a.gx[0];
  *cblk = r - *kz * a.gx[0];
  *src = 0;
  const int n_tiles = b.sched[1];
  if (u >= n_tiles) return false;
  // The list holds the wide experts' tiles, then the sched[2] one-tile thin
  // experts' (at most 32 rows); `order` places the thin ones in dispatch
  // order: 0 last, 1 first, 2 spread evenly among the wide ones.
  const int n_thin = b.sched[2], n_wide = n_tiles - n_thin;
  if (order == 1) {
    u += n_wide;
    if (u >= n_tiles) u -= n_tiles;
  } else if (order == 2 && n_thin > 0) {
    // slots [0, u) hold c(u) = floor(u * n_thin / n_tiles) thin tiles
    const int c0 = (int)((int64_t)u * n_thin / n_tiles);
    const int c1 = (int)((int64_t)(u + 1) * n_thin / n_tiles);
    u = c1 > c0 ? n_wide + c0 : u - c0;
  }
  const int4 t = reinterpret_cast<const int4*>(b.sched + sched_tiles_offset(b.E))[u];
  v->e = t.x;
  v->row0 = t.y;
  v->nrows = t.z;
  return true;
}

template <int MS>
constexpr int a_chunks() {
  return (MS * 32 + kChunkRows - 1) / kChunkRows;
}

// One tile: MS row subtiles of 32 (compile-time, so the accumulators stay in
// fixed registers), NS column subtiles of 32 per wave, P weight planes, K
// steps [k0, k1), weights in format FMT.
//
// Pipeline (one barrier per K step, two LDS buffers, register rings of DA
// activation and DB weight stages): at step s a wave decodes B(s), issues the
// global loads of A(s+DA) and B(s+DB), runs the MFMAs of step s, then writes
// A(s+1) into the idle LDS buffer.  Two workgroups share a CU, so one's
// decode, LDS traffic and barrier waits overlap the other's MFMAs.
// Scheduling barriers keep the compiler from sinking the loads below the
// MFMAs.  Loads past the last step re-read the last step (their data is never
// used), which keeps the loop free of branches around loads and accumulators.
template <int P, int NS, int MODE, int MS, int FMT>
__device__ __forceinline__ void gemm_tile(const TileView& tv, const GemmSrc& S, const GemmArgs& a,
                                          const uint16_t* const (&arow)[a_chunks<MS>()],
                                          char (*lds)[kBM * kPitch], const int* row_tok,
                                          const float* row_w, int cblk, int k0, int k1) {
  constexpr int NA = a_chunks<MS>();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 31, hf = lane >> 5;
  constexpr int WN = 32 * NS;
  constexpr int BN = kWaves * WN;
  const int col0 = cblk * BN + wave * WN;
  const int K = S.K, N = S.N;
  const int n = k1 - k0;  // steps of this workgroup

  // Weight pointers of this lane at step 0 (columns past N re-read valid
  // rows; they are never stored).  Row layout: row col0+32*ns+j, group
  // 2*step+hf, consecutive steps 2 groups apart.  Tiled layout: lane's 16
  // bytes of the 1 KB block (subtile, step), consecutive steps 1 KB apart.
  using SElem = std::conditional_t<FMT == kFmtMxfp4, uint8_t, uint16_t>;
  const u32x4_t* bq_ptr[NS][P];
  const SElem* bs_ptr[NS][P];
  const int64_t plane = (int64_t)N * (K / 2), splane = (int64_t)N * (K / 32);
  const int stride = S.tiled ? 64 : 2;  // per K step, in 16-byte / scale units
#pragma unroll
  for (int ns = 0; ns < NS; ++ns) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (S.tiled) {
        const int64_t blk = (int64_t)(min(col0 + ns * 32, N - 32) / 32) * (K / 64) + k0;
        bq_ptr[ns][p] = reinterpret_cast<const u32x4_t*>(S.q[p] + tv.e * plane + blk * 1024) + lane;
        bs_ptr[ns][p] = static_cast<const SElem*>(S.s[p]) + tv.e * splane + blk * 64 + lane;
      } else {
        const int row = min(col0 + ns * 32 + j, N - 1);
        bq_ptr[ns][p] = reinterpret_cast<const u32x4_t*>(S.q[p] + tv.e * plane + (int64_t)row * (K / 2)) +
                        hf + 2 * k0;
        bs_ptr[ns][p] = static_cast<const SElem*>(S.s[p]) + tv.e * splane + (int64_t)row * (K / 32) +
                        hf + 2 * k0;
      }
    }
  }
  auto b_load = [&](BStage<P, NS>& st, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int p = 0; p < P; ++p) {
        st.q[ns][p] = bq_ptr[ns][p][stride * s];
        st.s[ns][p] = bs_ptr[ns][p][stride * s];
      }
  };
  const int chunk = threadIdx.x & 7;
  auto a_load = [&](AStage<NA>& st, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NA; ++i)
      st.v[i] = reinterpret_cast<const u32x4_t*>(arow[i] + (int64_t)(k0 + s) * kKS)[chunk];
  };
  auto a_store = [&](const AStage<NA>& st, char* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int r = (threadIdx.x >> 3) + kChunkRows * i;
      *reinterpret_cast<u32x4_t*>(buf + r * kPitch + chunk * 16) = st.v[i];
    }
  };

  // MXFP4: each weight row's shift (see e8m0_f16_shifted), from the largest
  // finite exponent of the groups this workgroup contracts, agreed between
  // the lanes j and j + 32 that feed the same output column.
  int mx_shift[NS][P];
#pragma unroll
  for (int ns = 0; ns < NS; ++ns)
#pragma unroll
    for (int p = 0; p < P; ++p) {
      mx_shift[ns][p] = 0;
      if constexpr (FMT == kFmtMxfp4) {
        int m = -1;
        const SElem* sp = bs_ptr[ns][p];
#pragma unroll 8
        for (int s2 = 0; s2 < n; ++s2) {
          const int e = sp[stride * s2];
          m = (e != 255 && e > m) ? e : m;
        }
        m = max(m, __shfl_xor(m, 32, 64));
        mx_shift[ns][p] = mx_row_shift(m);
      }
    }

  f32x16_t acc[MS][NS][P];
#pragma unroll
  for (int m = 0; m < MS; ++m)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[m][ns][p][v] = 0.f;

  // Decoded weight operands: word d of a lane's 16 bytes feeds MFMA d.  The
  // group scale pairs of a stage first, then one word at a time.
  struct BScale {
    f16x2_t s2[NS][P], m8s2[NS][P];
  };
  auto scales = [&](const BStage<P, NS>& st) __attribute__((always_inline)) {
    BScale r;
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int p = 0; p < P; ++p) {
        _Float16 sc;
        if constexpr (FMT == kFmtMxfp4) sc = e8m0_f16_shifted(st.s[ns][p], mx_shift[ns][p]);
        else sc = __builtin_bit_cast(_Float16, (uint16_t)st.s[ns][p]);
        r.s2[ns][p] = f16x2_t{sc, sc};
        r.m8s2[ns][p] = r.s2[ns][p] * f16x2_t{(_Float16)-8.0f, (_Float16)-8.0f};
      }
    return r;
  };
  typedef f16x8_t BWord[NS][P];
  auto decode_word = [&](const BStage<P, NS>& st, const BScale& sc, int d, BWord& bw)
      __attribute__((always_inline)) {
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int p = 0; p < P; ++p) {
        if constexpr (FMT == kFmtMxfp4)
          bw[ns][p] = MS == 1 ? mx4_f16x8_cvt(st.q[ns][p][d], sc.s2[ns][p])
                              : mx4_f16x8(st.q[ns][p][d], sc.s2[ns][p]);
        else if constexpr (MS == 1)
          bw[ns][p] = q4_f16x8_cvt(st.q[ns][p][d], sc.s2[ns][p], sc.m8s2[ns][p]);
        else
          bw[ns][p] = q4_f16x8(st.q[ns][p][d], sc.s2[ns][p]);
      }
  };

  // Register rings: A(s) lives in as[s % DA] from its load (step s-DA)
  // until its LDS write (end of step s-1); B(s) lives in bs[s % DB] from its
  // load (step s-DB) until the start of step s, where it is copied out and
  // its slot refilled.
  constexpr int DA = MOE_GEMM_DA, DB = MOE_GEMM_DB;
  constexpr int U = lcm_c(DA, DB);
  AStage<NA> as[DA];
  BStage<P, NS> bs[DB];

  // One K step at ring phase u (s % U == u).  Word 0 is decoded before the
  // MFMAs (or, with kAhead, under the previous step's last MFMAs, into
  // bw[0], which word 2's MFMAs no longer read); word d + 1 is decoded while
  // the MFMAs of word d run, so the decode's VALU work overlaps the matrix
  // pipe inside one wave.
  constexpr bool kAhead = FMT == kFmtInt4 && (MOE_GEMM_W0_AHEAD & (MODE == 1 ? 2 : 1)) != 0;
  BWord bw[2];
  auto step = [&](int s, auto uc) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value;
    const BStage<P, NS> cur = bs[u % DB];
    const BScale sc = scales(cur);
    if constexpr (!kAhead) decode_word(cur, sc, 0, bw[0]);
    b_load(bs[u % DB], min(s + DB, n - 1));
    a_load(as[u % DA], min(s + DA, n - 1));
    __builtin_amdgcn_sched_barrier(0);
    const char* cur_lds = lds[s & 1];
    static_for<4>([&](auto dc) __attribute__((always_inline)) {
      constexpr int d = decltype(dc)::value;
      if constexpr (d < 3) {
        decode_word(cur, sc, d + 1, bw[(d + 1) & 1]);
      } else if constexpr (kAhead) {
        // word 0 of step s + 1 from its ring slot (loaded a step ago; a
        // past-the-end step re-reads the last one and is never used)
        const BStage<P, NS>& nxt = bs[(u + 1) % DB];
        decode_word(nxt, scales(nxt), 0, bw[0]);
      }
#pragma unroll
      for (int m = 0; m < MS; ++m) {
        const f16x8_t af =
            *reinterpret_cast<const f16x8_t*>(cur_lds + (m * 32 + j) * kPitch + hf * 64 + 16 * d);
#pragma unroll
        for (int ns = 0; ns < NS; ++ns)
#pragma unroll
          for (int p = 0; p < P; ++p)
            acc[m][ns][p] =
                __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bw[d & 1][ns][p], acc[m][ns][p], 0, 0, 0);
      }
    });
    __builtin_amdgcn_sched_barrier(0);
    a_store(as[(u + 1) % DA], lds[(s + 1) & 1]);
    __syncthreads();
  };

  static_for<DB>([&](auto i) __attribute__((always_inline)) {
    b_load(bs[decltype(i)::value], min((int)decltype(i)::value, n - 1));
  });
  static_for<DA>([&](auto i) __attribute__((always_inline)) {
    a_load(as[decltype(i)::value], min((int)decltype(i)::value, n - 1));
  });
  a_store(as[0], lds[0]);
  if constexpr (kAhead) decode_word(bs[0], scales(bs[0]), 0, bw[0]);
  __syncthreads();
  int s = 0;
  for (; s + U <= n; s += U)
    static_for<U>([&](auto i) __attribute__((always_inline)) { step(s + decltype(i)::value, i); });
  if (s < n)
    static_for<U>([&](auto i) __attribute__((always_inline)) {
      if (s + decltype(i)::value < n) step(s + decltype(i)::value, i);
    });

  // Epilogue.  Lane (j, hf) holds column col0 + ns*32 + j, rows
  // m*32 + 8*(v/4) + 4*hf + v%4 of the tile.
#pragma unroll
  for (int m = 0; m < MS; ++m) {
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      const int col = col0 + ns * 32 + j;
      if (col >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = m * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
        if (i >= tv.nrows) continue;
        if (MODE == 0) {
          float g = acc[m][ns][0][v], u = acc[m][ns][P - 1][v];
          if constexpr (FMT == kFmtMxfp4) {
            g = ldexpf(g, mx_shift[ns][0]);
            u = ldexpf(u, mx_shift[ns][P - 1]);
          }
          const float hv = g / (1.0f + __expf(-g)) * u;
          const _Float16 hh = (_Float16)hv;
          S.hout[(int64_t)(tv.row0 + i) * N + perm_col(col)] = __builtin_bit_cast(uint16_t, hh);
        } else {
          const float o = FMT == kFmtMxfp4 ? ldexpf(acc[m][ns][0][v], mx_shift[ns][0])
                                           : acc[m][ns][0][v];
          unsafeAtomicAdd(&a.y[(int64_t)row_tok[i] * a.H + col], row_w[i] * o);
        }
      }
    }
  }
}

}  // namespace

// P planes (2 = gate and up, 1 = down), NS 32-column subtiles per wave, FMT
// the weight format.
// MODE 0: gate/up -> h16 = fp16(silu(g) * u) at the tile's rows.
// MODE 1: down    -> y[token] += weight * acc (fp32 atomics), K split over
//                    blockIdx.z into a.ksplit ranges.
template <int P, int NS, int MODE, int FMT>
__global__ __launch_bounds__(kThreads, MOE_GEMM_OCC) void gemm_kernel(Buckets b, GemmArgs a) {
  if (MODE == 0 && a.y_zero) {
    // every workgroup of the launch, tile or not, clears its share of y
    const int64_t nthr = (int64_t)gridDim.x * gridDim.y * kThreads;
    const int64_t gid = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * kThreads + threadIdx.x;
    float4* y4 = reinterpret_cast<float4*>(a.y_zero);
    for (int64_t i = gid; i < a.y_elems / 4; i += nthr) y4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  TileView tv;
  int src = 0, cblk = 0, kz = 0;
  if (!tile_of(b, a, &tv, &src, &cblk, &kz,
               MODE == 0 ? MOE_GEMM_THIN_ORDER_GU : MOE_GEMM_THIN_ORDER_DN))
    return;
  const GemmSrc S = src ? a.src[1] : a.src[0];

  __shared__ __attribute__((aligned(16))) char lds[2][kBM * kPitch];
  __shared__ int row_tok[kBM];
  __shared__ float row_w[kBM];

  // Destination token and combine weight of each tile row (down pass).
  if (MODE == 1 && threadIdx.x < kBM) {
    const int i = threadIdx.x;
    int tok = 0;
    float wt = 0.f;
    if (i < tv.nrows) {
      const int r = tv.row0 + i;
      if (src) {
        tok = r;
        wt = a.gate_logit ? sigmoidf_acc(a.gate_logit[(int64_t)r * a.gate_ld]) : 1.0f;
      } else {
        const int s = b.sorted[r];
        tok = s / b.k;
        wt = a.w[s];
      }
    }
    row_tok[i] = tok;
    row_w[i] = wt;
  }

  // K range of this workgroup
  const int nks = S.K / kKS;
  int k0 = 0, k1 = nks;
  if (MODE == 1) {
    const int ks = S.ksplit;
    k0 = (int)((int64_t)nks * kz / ks);
    k1 = (int)((int64_t)nks * (kz + 1) / ks);
  }

  // Source row of each activation chunk this thread loads; rows past the
  // tile re-read its last row (their results are never stored).
  auto src_row = [&](int i) -> const uint16_t* {
    const int r = tv.row0 + min(i, tv.nrows - 1);
    int64_t row = r;
    if (MODE == 0 && !src) row = b.sorted[r] / b.k;
    return S.act + row * S.K;
  };
  const int r0 = threadIdx.x >> 3;
  const int msub = (tv.nrows + 31) >> 5;
  static_for<4>([&](auto c) __attribute__((always_inline)) {
    constexpr int MS = decltype(c)::value + 1;
    constexpr int NA = a_chunks<MS>();
    if (msub == MS) {
      const uint16_t* rows[NA];
#pragma unroll
      for (int i = 0; i < NA; ++i) rows[i] = src_row(r0 + kChunkRows * i);
      gemm_tile<P, NS, MODE, MS, FMT>(tv, S, a, rows, lds, row_tok, row_w, cblk, k0, k1);
    }
  });
}

namespace {

constexpr int kDownNS = MOE_GEMM_DN_NS;
constexpr int kGateUpNS = MOE_GEMM_GU_NS;

// K ranges for one source of the down pass: about equal work per workgroup,
// enough workgroups to cover the chip twice, and at least 16 K steps each
// (shorter ranges spend more on the pipeline's ramp and the atomic epilogue
// than they gain in parallelism).
int down_split(int nks, int64_t total_steps) {
  const int64_t target = std::max<int64_t>(16, total_steps / 512);
  int s = (int)((nks + target - 1) / target);
  s = std::min(s, std::max(1, nks / 16));
  return std::max(1, std::min(s, 64));
}

// At least ceil(slots/128) routed tiles; about half the experts add a short one.
int64_t routed_tile_estimate(const Buckets& b) {
  const int64_t slots = (int64_t)b.max_rows * b.k;
  return (slots + kBM - 1) / kBM + std::min<int64_t>(b.E, slots) / 2;
}

template <int P, int NS, int MODE>
hipError_t launch_tiles(const Buckets& b, int max_tiles, GemmArgs a, int fmt, const Launch& L) {
  constexpr int BN = kWaves * 32 * NS;
  a.gx[0] = (a.src[0].N + BN - 1) / BN;
  a.gx[1] = a.shared_tiles > 0 ? (a.src[1].N + BN - 1) / BN : 1;
  a.src[0].ksplit = std::max(a.src[0].ksplit, 1);
  a.src[1].ksplit = std::max(a.src[1].ksplit, 1);
  const int64_t wgs = (int64_t)a.shared_tiles * a.gx[1] * a.src[1].ksplit +
                      (int64_t)max_tiles * a.gx[0] * a.src[0].ksplit;
  if (wgs < 1 || wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs);
  if (fmt == kFmtMxfp4)
    MOE_LAUNCH(L, (gemm_kernel<P, NS, MODE, kFmtMxfp4>), grid, dim3(kThreads), 0, b, a);
  else
    MOE_LAUNCH(L, (gemm_kernel<P, NS, MODE, kFmtInt4>), grid, dim3(kThreads), 0, b, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_gate_up(const Buckets& b, int max_tiles, const uint16_t* x16, int H,
                               int I, const uint8_t* gq, const void* gs,
                               const uint8_t* uq, const void* us, uint16_t* h16,
                               const SharedGemm* shared, float* y_zero, int64_t y_elems,
                               bool tiled, int fmt, const Launch& L) {
  GemmArgs a{};
  a.src[0].tiled = a.src[1].tiled = tiled ? 1 : 0;
  a.y_zero = y_zero;
  a.y_elems = y_elems;
  GemmSrc& r = a.src[0];
  r.act = x16;
  r.K = H;
  r.N = I;
  r.q[0] = gq;
  r.s[0] = gs;
  r.q[1] = uq;
  r.s[1] = us;
  r.hout = h16;
  r.ksplit = 1;
  if (shared) {
    GemmSrc& sh = a.src[1];
    sh.act = x16;
    sh.K = H;
    sh.N = shared->SI;
    sh.q[0] = shared->q[0];
    sh.s[0] = shared->s[0];
    sh.q[1] = shared->q[1];
    sh.s[1] = shared->s[1];
    sh.hout = shared->h16;
    sh.ksplit = 1;
    a.shared_T = shared->T;
    a.shared_rows = tiled ? MOE_GEMM_SHARED_ROWS_GU : kBM;
    a.shared_tiles = (shared->T + a.shared_rows - 1) / a.shared_rows;
  }
  a.H = H;
  return launch_tiles<2, kGateUpNS, 0>(b, max_tiles, a, fmt, L);
}

hipError_t launch_gemm_down(const Buckets& b, int max_tiles, const uint16_t* h16, int H, int I,
                            const uint8_t* dq, const void* ds, const float* w, float* y,
                            const SharedGemm* shared, bool tiled, int fmt, const Launch& L) {
  GemmArgs a{};
  a.src[0].tiled = a.src[1].tiled = tiled ? 1 : 0;
  GemmSrc& r = a.src[0];
  r.act = h16;
  r.K = I;
  r.N = H;
  r.q[0] = r.q[1] = dq;
  r.s[0] = r.s[1] = ds;
  a.w = w;
  a.y = y;
  a.H = H;
  constexpr int BN = kWaves * 32 * kDownNS;
  const int gx = (H + BN - 1) / BN;
  const int64_t est = routed_tile_estimate(b);
  int64_t total = est * gx * (I / kKS);
  if (shared) {
    GemmSrc& sh = a.src[1];
    sh.act = shared->h16;
    sh.K = shared->SI;
    sh.N = H;
    sh.q[0] = sh.q[1] = shared->q[2];
    sh.s[0] = sh.s[1] = shared->s[2];
    a.shared_T = shared->T;
    a.shared_rows = tiled ? MOE_GEMM_SHARED_ROWS_DN : kBM;
    a.shared_tiles = (shared->T + a.shared_rows - 1) / a.shared_rows;
    a.gate_logit = shared->gate_logit;
    a.gate_ld = shared->gate_ld;
    total += (int64_t)a.shared_tiles * gx * (shared->SI / kKS);
  }
  r.ksplit = down_split(I / kKS, total);
  if (shared) a.src[1].ksplit = down_split(shared->SI / kKS, total);
  return launch_tiles<1, kDownNS, 1>(b, max_tiles, a, fmt, L);
}

}  // namespace moe
