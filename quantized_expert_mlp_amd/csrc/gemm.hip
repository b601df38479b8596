// Grouped int4 GEMM on fp16 MFMA for prefill-sized buckets.
//
// Sources: the dasLLAMA vulkan PR #3988 routed block (bucket rows gathered
// through the slot map into expert tiles, an upper-bound dispatch whose
// surplus workgroups return at once, the act step between gate/up and down,
// the combine reading each slot's row through the map; the shared expert as
// one more region over every row with an identity map, weighted by the
// sigmoid of its gate logit) and the colibri PR #418 int4 format (nibble - 8,
// one fp16 scale per 32 inputs).
//
// gfx950 design.  A workgroup (4 waves) owns one row tile of up to 128 bucket
// rows and a block of output columns; waves split the columns, so each wave
// decodes its own weight fragment straight from a 128-bit global load into
// MFMA operand registers (no LDS round trip for weights), while the activation
// tile - shared by the four waves - is staged through LDS, double-buffered,
// one barrier per 64-deep K step.  The MFMA is v_mfma_f32_32x32x16_f16:
//   A (32 rows x 16 k)  lane l: row l%32, k 8*(l/32)..+7  (activations)
//   B (16 k x 32 cols)  lane l: col l%32, k 8*(l/32)..+7  (weights)
//   D (32 x 32, fp32)   lane l: col l%32, rows 8*(v/4) + 4*(l/32) + v%4.
// The weight operand is the exact dequantised value (nibble-8)*scale rounded
// once to fp16; fp16 and bf16 MFMA have the same peak on gfx950, and fp16's
// 11-bit significand keeps the layer within its tolerance where bf16 would
// not.  Activations are fp16 copies stored with each block of 8 in the order
// 0,4,1,5,2,6,3,7, matching the nibble pairing of the decode.
//
// K mapping inside one 64-deep step: lane (j, hf) = (l%32, l/32) loads the 16
// bytes of scale group 2*step + hf of weight row j; packed word d of it feeds
// MFMA d.  MFMA d therefore contracts k = 32*hf + 8*d + {0..7}: its A operand
// is the 16 bytes at k offset 32*hf + 8*d of the LDS activation row.
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kBM = kGemmTileRows;    // 128 rows per tile
constexpr int kKS = 64;               // K per step
constexpr int kPitch = kKS * 2 + 16;  // LDS row pitch in bytes (padding breaks bank conflicts)

struct TileView {
  int e, row0, nrows;
};

__device__ __forceinline__ bool tile_of(const Buckets& b, TileView* v) {
  const int u = blockIdx.y;
  if (b.shared_T > 0) {
    v->e = 0;
    v->row0 = u * kBM;
    v->nrows = min(kBM, b.shared_T - v->row0);
    return v->nrows > 0;
  }
  if (u >= b.sched[1]) return false;
  const int4 t = reinterpret_cast<const int4*>(b.sched + sched_tiles_offset(b.E))[u];
  v->e = t.x;
  v->row0 = t.y;
  v->nrows = t.z;
  return true;
}

// Row-major fp16 position of logical column j in the permuted-by-8 layout.
__device__ __forceinline__ int perm_col(int j) { return (j & ~7) | perm8_pos(j & 7); }

// Stage one 128 x 64 fp16 activation tile (K step ks) into LDS.  Thread t
// copies 64 bytes: row t/2, half t%2.  Rows past the tile are zero.
struct AStage {
  uint4 v[4];
};

__device__ __forceinline__ void a_load(AStage& s, const uint16_t* const* rowp, int K, int ks) {
  const int half = threadIdx.x & 1;
  const uint16_t* p = rowp[threadIdx.x >> 1];
  if (p) {
    const uint4* src = reinterpret_cast<const uint4*>(p + (int64_t)ks * kKS + half * 32);
#pragma unroll
    for (int c = 0; c < 4; ++c) s.v[c] = src[c];
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) s.v[c] = make_uint4(0, 0, 0, 0);
  }
  (void)K;
}

__device__ __forceinline__ void a_store(const AStage& s, char* lds) {
  const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
  uint4* dst = reinterpret_cast<uint4*>(lds + row * kPitch + half * 64);
#pragma unroll
  for (int c = 0; c < 4; ++c) dst[c] = s.v[c];
}

}  // namespace

// P planes (2 = gate and up, 1 = down), NS 32-column subtiles per wave.
// MODE 0: gate/up -> h16 = fp16(silu(g) * u) at the tile's rows.
// MODE 1: down    -> y[token] += weight * acc (fp32 atomics).
template <int P, int NS, int MODE>
__global__ __launch_bounds__(256) void gemm_kernel(
    Buckets b, const uint16_t* __restrict__ act, int K, int N, const uint8_t* __restrict__ q0,
    const uint16_t* __restrict__ s0, const uint8_t* __restrict__ q1,
    const uint16_t* __restrict__ s1, uint16_t* __restrict__ hout, const float* __restrict__ w,
    const float* __restrict__ gate_logit, int gate_ld, float* __restrict__ y, int H, int ldh) {
  TileView tv;
  if (!tile_of(b, &tv)) return;

  __shared__ __attribute__((aligned(16))) char lds[2][kBM * kPitch];
  __shared__ const uint16_t* rowp[kBM];
  __shared__ int row_tok[kBM];
  __shared__ float row_w[kBM];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 31, hf = lane >> 5;
  constexpr int WN = 32 * NS;      // columns per wave
  constexpr int BN = 4 * WN;       // columns per workgroup
  const int col0 = blockIdx.x * BN + wave * WN;

  // Per-row sources (activation row pointer) and, for the down pass, the
  // destination token and combine weight.
  if (threadIdx.x < kBM) {
    const int i = threadIdx.x;
    const uint16_t* p = nullptr;
    int tok = -1;
    float wt = 0.f;
    if (i < tv.nrows) {
      const int r = tv.row0 + i;
      if (b.shared_T > 0) {
        tok = r;
        wt = (MODE == 1 && gate_logit) ? sigmoidf_acc(gate_logit[(int64_t)r * gate_ld]) : 1.0f;
      } else {
        const int s = b.sorted[r];
        tok = s / b.k;
        wt = (MODE == 1) ? w[s] : 1.0f;
      }
      p = (MODE == 0) ? act + (int64_t)tok * K : act + (int64_t)r * K;
    }
    rowp[i] = p;
    row_tok[i] = tok;
    row_w[i] = wt;
  }
  __syncthreads();

  const int64_t plane = (int64_t)N * (K / 2), splane = (int64_t)N * (K / 32);
  const uint8_t* qp[P];
  const uint16_t* sp[P];
  qp[0] = q0 + tv.e * plane;
  sp[0] = s0 + tv.e * splane;
  if (P > 1) {
    qp[P - 1] = q1 + tv.e * plane;
    sp[P - 1] = s1 + tv.e * splane;
  }

  // Weight row of this lane for subtile ns; columns past N read nothing.
  int wrow[NS];
  bool wvalid[NS];
#pragma unroll
  for (int ns = 0; ns < NS; ++ns) {
    wrow[ns] = col0 + ns * 32 + j;
    wvalid[ns] = wrow[ns] < N;
  }
  // Row tiles of 32 that hold at least one real row (wave-uniform).
  const int msub = (tv.nrows + 31) / 32;

  f32x16_t acc[4][NS][P];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[m][ns][p][v] = 0.f;

  const int nks = K / kKS;
  uint4 bq[NS][P];
  uint16_t bs[NS][P];
  auto b_load = [&](int ks) {
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int p = 0; p < P; ++p) {
        if (wvalid[ns]) {
          const int g = 2 * ks + hf;
          bq[ns][p] = *reinterpret_cast<const uint4*>(qp[p] + (int64_t)wrow[ns] * (K / 2) + 16 * g);
          bs[ns][p] = sp[p][(int64_t)wrow[ns] * (K / 32) + g];
        } else {
          bq[ns][p] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
          bs[ns][p] = 0;
        }
      }
  };

  AStage as;
  a_load(as, rowp, K, 0);
  b_load(0);
  a_store(as, lds[0]);
  __syncthreads();

  for (int ks = 0; ks < nks; ++ks) {
    // decode this step's weights into MFMA operands
    f16x8_t bf[NS][P][4];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const _Float16 sc = __builtin_bit_cast(_Float16, bs[ns][p]);
        const f16x2_t s2 = {sc, sc};
        bf[ns][p][0] = q4_f16x8(bq[ns][p].x, s2);
        bf[ns][p][1] = q4_f16x8(bq[ns][p].y, s2);
        bf[ns][p][2] = q4_f16x8(bq[ns][p].z, s2);
        bf[ns][p][3] = q4_f16x8(bq[ns][p].w, s2);
      }
    const bool more = ks + 1 < nks;
    if (more) {
      a_load(as, rowp, K, ks + 1);
      b_load(ks + 1);
    }
    const char* cur = lds[ks & 1];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m < msub) {
        const char* arow = cur + (m * 32 + j) * kPitch + hf * 64;
        f16x8_t af[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) af[d] = *reinterpret_cast<const f16x8_t*>(arow + 16 * d);
#pragma unroll
        for (int ns = 0; ns < NS; ++ns)
#pragma unroll
          for (int p = 0; p < P; ++p)
#pragma unroll
            for (int d = 0; d < 4; ++d)
              acc[m][ns][p] =
                  __builtin_amdgcn_mfma_f32_32x32x16_f16(af[d], bf[ns][p][d], acc[m][ns][p], 0, 0, 0);
      }
    }
    if (more) a_store(as, lds[(ks + 1) & 1]);
    __syncthreads();
  }

  // Epilogue.  Lane (j, hf) holds column col0 + ns*32 + j, rows
  // m*32 + 8*(v/4) + 4*hf + v%4 of the tile.
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (m >= msub) continue;
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      const int col = col0 + ns * 32 + j;
      if (col >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = m * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
        if (i >= tv.nrows) continue;
        if (MODE == 0) {
          const float g = acc[m][ns][0][v], u = acc[m][ns][P - 1][v];
          const float hv = g / (1.0f + __expf(-g)) * u;
          const _Float16 hh = (_Float16)hv;
          hout[(int64_t)(tv.row0 + i) * ldh + perm_col(col)] = __builtin_bit_cast(uint16_t, hh);
        } else {
          unsafeAtomicAdd(&y[(int64_t)row_tok[i] * H + col], row_w[i] * acc[m][ns][0][v]);
        }
      }
    }
  }
}

hipError_t launch_gemm_gate_up(const Buckets& b, int max_tiles, const uint16_t* x16, int H,
                               int I, const uint8_t* gq, const uint16_t* gs,
                               const uint8_t* uq, const uint16_t* us, uint16_t* h16,
                               const Launch& L) {
  constexpr int BN = 4 * 32 * 1;
  dim3 grid((I + BN - 1) / BN, max_tiles);
  MOE_LAUNCH(L, (gemm_kernel<2, 1, 0>), grid, dim3(256), 0, b, x16, H, I, gq, gs, uq, us,
                     h16, nullptr, nullptr, 0, nullptr, H, I);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const Buckets& b, int max_tiles, const uint16_t* h16, int H, int I,
                            const uint8_t* dq, const uint16_t* ds, const float* w,
                            const float* gate_logit, int gate_ld, float* y, const Launch& L) {
  constexpr int BN = 4 * 32 * 2;
  dim3 grid((H + BN - 1) / BN, max_tiles);
  MOE_LAUNCH(L, (gemm_kernel<1, 2, 1>), grid, dim3(256), 0, b, h16, I, H, dq, ds, dq, ds,
                     nullptr, w, gate_logit, gate_ld, y, H, 0);
  return hipGetLastError();
}

}  // namespace moe
