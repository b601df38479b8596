// libmoe C ABI: argument checks, workspace layout and the launch sequence.
// The declarations and their contracts are in include/moe.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "moe.h"
#include "kernels.h"

// The workspace of moe_layer_static: device memory owned by the library, one
// copy per GPU (each device that runs the library holds it until the process
// ends).  Host code never passes this name to a kernel: its host-side symbol
// is a stand-in, not a device address; the device address comes from
// hipGetSymbolAddress, once per device (static_scratch below).
static __device__ __align__(256) char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

using moe::Buckets;

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Router variant checks: a known score function, an aligned bias, a grouping
// that divides the experts into at most kMaxGroups groups whose kept part
// holds at least k experts, and top-p only with the plain softmax router.
int check_router(int32_t score, const float* bias, float top_p, int32_t n_group,
                 int32_t topk_group, int32_t E, int32_t k) {
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (bias && !aligned(bias, 4)) return MOE_ERR_INVALID_ARG;
  if (n_group < 0) return MOE_ERR_INVALID_ARG;
  if (n_group > 1) {
    if (n_group > moe::kMaxGroups) return MOE_ERR_UNSUPPORTED;
    if (E % n_group || topk_group < 1 || topk_group > n_group ||
        (int64_t)topk_group * (E / n_group) < k)
      return MOE_ERR_INVALID_ARG;
  }
  const bool variant = score != MOE_SCORE_SOFTMAX || bias != nullptr || n_group > 1;
  if (variant && top_p > 0.0f && top_p < 1.0f) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe::RouterSpec router_spec(const moe_shape* sh) {
  return moe::RouterSpec{sh->route_scale, sh->top_p,  sh->score,
                         sh->select_bias, sh->n_group, sh->topk_group};
}

// Shape checks shared by every entry point that takes a moe_shape.
int check_shape(const moe_shape* sh) {
  if (!sh) return MOE_ERR_INVALID_ARG;
  if (sh->T < 1 || sh->H < 1 || sh->E < 1 || sh->k < 1 || sh->I < 1 || sh->SI < 0)
    return MOE_ERR_INVALID_ARG;
  if (sh->k > sh->E) return MOE_ERR_INVALID_ARG;
  if (sh->group != 32) return MOE_ERR_UNSUPPORTED;
  if (sh->path < MOE_PATH_AUTO || sh->path > MOE_PATH_GEMM) return MOE_ERR_INVALID_ARG;
  if (sh->layout != MOE_LAYOUT_ROWS && sh->layout != MOE_LAYOUT_TILED) return MOE_ERR_INVALID_ARG;
  if (sh->format != MOE_FORMAT_INT4 && sh->format != MOE_FORMAT_MXFP4) return MOE_ERR_INVALID_ARG;
  if (sh->E > 256 || sh->k > 64) return MOE_ERR_UNSUPPORTED;
  if (sh->H % 64 || sh->I % 64 || sh->SI % 64) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)sh->T * sh->k >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)sh->T * sh->H >= (int64_t)1 << 40) return MOE_ERR_UNSUPPORTED;
  return check_router(sh->score, sh->select_bias, sh->top_p, sh->n_group, sh->topk_group, sh->E,
                      sh->k);
}

bool gemv_ok(const moe_shape* sh) {
  if (sh->layout == MOE_LAYOUT_TILED)
    return moe::gemv_tiled_supported(sh->H) && moe::gemv_tiled_supported(sh->I) &&
           (sh->SI == 0 || moe::gemv_tiled_supported(sh->SI));
  return moe::gemv_supported(sh->H) && moe::gemv_supported(sh->I) &&
         (sh->SI == 0 || moe::gemv_supported(sh->SI));
}

// The grouped MFMA GEMM is taken when an expert's bucket is expected to hold
// at least 8 rows (slots / E >= 8), or when the GEMV cannot serve the shape.
// Tiled planes take the GEMV only for the few tokens its fused routing
// serves (beyond that the MFMA GEMM reads them faster).
int pick_gemm(const moe_shape* sh, bool* gemm) {
  const int64_t slots = (int64_t)sh->T * sh->k;
  switch (sh->path) {
    case MOE_PATH_GEMV:
      if (!gemv_ok(sh)) return MOE_ERR_UNSUPPORTED;
      *gemm = false;
      return MOE_OK;
    case MOE_PATH_GEMM:
      *gemm = true;
      return MOE_OK;
    default:
      if (sh->layout == MOE_LAYOUT_TILED)
        *gemm = !gemv_ok(sh) || sh->T > moe::kFusedRouteMaxT || slots > moe::kFusedRouteMaxSlots;
      else
        *gemm = !gemv_ok(sh) || slots >= 8 * (int64_t)sh->E;
      return MOE_OK;
  }
}

struct Layout {
  size_t logits, gate, idx, w, off, sorted, row_of, sched, pscratch, x16, h, hs, total;
  int ld;  // logits row stride in the workspace (E, or E+1 with a gate column)
};

Layout make_layout(const moe_shape* sh, bool gemm) {
  const int64_t T = sh->T, E = sh->E, slots = T * sh->k;
  Layout L{};
  size_t p = 0;
  auto take = [&](size_t bytes) {
    const size_t at = p;
    p += align_up(bytes ? bytes : 1);
    return at;
  };
  L.ld = (int)E + 1;
  L.logits = take(sizeof(float) * T * (E + 1));
  L.gate = take(sizeof(float) * T);
  L.idx = take(sizeof(int32_t) * slots);
  L.w = take(sizeof(float) * slots);
  L.off = take(sizeof(int32_t) * (E + 2));
  L.sorted = take(sizeof(int32_t) * slots);
  L.row_of = take(sizeof(int32_t) * slots);
  L.sched = take(sizeof(int32_t) * moe::sched_words(slots, (int)E));
  L.pscratch = take(sizeof(int32_t) * moe::permute_scratch_words(slots, (int)E));
  L.x16 = take(gemm ? sizeof(uint16_t) * T * sh->H : 0);
  const size_t act = 2;  // hidden rows are fp16 on both paths
  L.h = take(act * slots * sh->I);
  L.hs = take(act * T * sh->SI);
  L.total = p;
  return L;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Device address of the static scratch on the current device, looked up on
// the first call made with that device current and kept per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// Optional per-stage events (moe_layer_profiled): stage i's kernel is launched
// with events[2i] / events[2i+1] recorded at its start and end; a stage a call
// does not run gets both events recorded back to back, so every pair is valid.
// ran (nullable, host): ran[i] is set to 1 for a stage whose kernel is
// launched, 0 for one the call skips.
struct Stages {
  void* const* ev;
  hipStream_t st;
  int32_t* ran = nullptr;
  moe::Launch at(int i) const {
    moe::Launch L{st};
    if (ev) {
      L.start = reinterpret_cast<hipEvent_t>(ev[2 * i]);
      L.stop = reinterpret_cast<hipEvent_t>(ev[2 * i + 1]);
    }
    if (ran) ran[i] = 1;
    return L;
  }
  bool skip(int i) const {
    if (ran) ran[i] = 0;
    if (!ev) return true;
    return hipEventRecord(reinterpret_cast<hipEvent_t>(ev[2 * i]), st) == hipSuccess &&
           hipEventRecord(reinterpret_cast<hipEvent_t>(ev[2 * i + 1]), st) == hipSuccess;
  }
};

bool plane_ok(const moe_q4& p) {
  return p.q && p.s && aligned(p.q, 16) && aligned(p.s, 16);
}

// Expert MLPs over the routed buckets (and the shared expert when given).
// x16_ready: the MFMA path's fp16 activation copy was written already (by the
// router logits launch).  accumulate: add into y as it is (the residual)
// instead of clearing it first.
int run_mlp(const moe_shape* sh, bool gemm, const Layout& L, void* ws, const uint16_t* x,
            const int32_t* off, const int32_t* sorted, const float* w, moe_q4 gate, moe_q4 up,
            moe_q4 down, const moe_q4* shared, const float* gate_logit, int gate_ld, float* y,
            hipStream_t st, const Stages& sg, const moe::RouteArgs* route = nullptr,
            bool x16_ready = false, bool accumulate = false) {
  const int T = sh->T, H = sh->H, I = sh->I, E = sh->E, k = sh->k;
  const int64_t slots = (int64_t)T * k;
  const int32_t* sched = at<int32_t>(ws, L.sched);
  Buckets routed{off, sorted, sched, k, 0, T, E};
  Buckets sharedb{nullptr, nullptr, nullptr, 1, T, T, 1};
  const int64_t y_elems = (int64_t)T * H;
  float* y_zero = accumulate ? nullptr : y;
  const int fmt = sh->format == MOE_FORMAT_MXFP4 ? moe::kFmtMxfp4 : moe::kFmtInt4;
  hipError_t err;
  if (!gemm) {
    uint16_t* h = at<uint16_t>(ws, L.h);
    uint16_t* hs = at<uint16_t>(ws, L.hs);
    const int max_buckets = (int)(slots < E ? slots : E);
    if (!sg.skip(MOE_STAGE_ACTIVATIONS)) return MOE_ERR_HIP;
    const bool tiled = sh->layout == MOE_LAYOUT_TILED;
    auto gate_up = tiled ? moe::launch_gemv_tiled_gate_up : moe::launch_gemv_gate_up;
    auto down_ = tiled ? moe::launch_gemv_tiled_down : moe::launch_gemv_down;
    err = gate_up(routed, max_buckets, x, H, I, gate.q, gate.s, up.q, up.s, h, y_zero, y_elems, fmt,
                  sg.at(MOE_STAGE_GATE_UP), route);
    if (err != hipSuccess) return MOE_ERR_HIP;
    if (shared) {
      err = gate_up(sharedb, 1, x, H, sh->SI, shared[0].q, shared[0].s, shared[1].q, shared[1].s,
                    hs, nullptr, 0, fmt, sg.at(MOE_STAGE_SHARED_GATE_UP), nullptr);
      if (err != hipSuccess) return MOE_ERR_HIP;
    } else if (!sg.skip(MOE_STAGE_SHARED_GATE_UP)) {
      return MOE_ERR_HIP;
    }
    err = down_(routed, max_buckets, h, H, I, down.q, down.s, w, nullptr, 0, y, fmt,
                sg.at(MOE_STAGE_DOWN));
    if (err != hipSuccess) return MOE_ERR_HIP;
    if (shared) {
      err = down_(sharedb, 1, hs, H, sh->SI, shared[2].q, shared[2].s, nullptr, gate_logit,
                  gate_ld, y, fmt, sg.at(MOE_STAGE_SHARED_DOWN));
      if (err != hipSuccess) return MOE_ERR_HIP;
    } else if (!sg.skip(MOE_STAGE_SHARED_DOWN)) {
      return MOE_ERR_HIP;
    }
    return MOE_OK;
  }
  uint16_t* x16 = at<uint16_t>(ws, L.x16);
  uint16_t* h16 = at<uint16_t>(ws, L.h);
  uint16_t* hs16 = at<uint16_t>(ws, L.hs);
  const int max_tiles = (int)moe::sched_max_tiles(slots, E);
  // the shared expert rides in the routed launches as extra tiles
  moe::SharedGemm sgm{};
  if (shared) {
    sgm.T = T;
    sgm.SI = sh->SI;
    for (int i = 0; i < 3; ++i) {
      sgm.q[i] = shared[i].q;
      sgm.s[i] = shared[i].s;
    }
    sgm.h16 = hs16;
    sgm.gate_logit = gate_logit;
    sgm.gate_ld = gate_ld;
  }
  const moe::SharedGemm* sgp = shared ? &sgm : nullptr;
  if (x16_ready) {
    if (!sg.skip(MOE_STAGE_ACTIVATIONS)) return MOE_ERR_HIP;
  } else {
    err = moe::launch_convert_x16(x, T, H, x16, sg.at(MOE_STAGE_ACTIVATIONS));
    if (err != hipSuccess) return MOE_ERR_HIP;
  }
  const bool tiled = sh->layout == MOE_LAYOUT_TILED;
  err = moe::launch_gemm_gate_up(routed, max_tiles, x16, H, I, gate.q, gate.s, up.q, up.s, h16,
                                 sgp, y_zero, y_elems, tiled, fmt, sg.at(MOE_STAGE_GATE_UP));
  if (err != hipSuccess) return MOE_ERR_HIP;
  if (!sg.skip(MOE_STAGE_SHARED_GATE_UP)) return MOE_ERR_HIP;
  err = moe::launch_gemm_down(routed, max_tiles, h16, H, I, down.q, down.s, w, y, sgp, tiled,
                              fmt, sg.at(MOE_STAGE_DOWN));
  if (err != hipSuccess) return MOE_ERR_HIP;
  if (!sg.skip(MOE_STAGE_SHARED_DOWN)) return MOE_ERR_HIP;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch error";
    case MOE_ERR_SCRATCH_LIMIT: return "shape needs more than the static scratch";
    default: return "unknown status";
  }
}

size_t moe_workspace_bytes(const moe_shape* sh) {
  if (check_shape(sh) != MOE_OK) return 0;
  bool gemm = false;
  if (pick_gemm(sh, &gemm) != MOE_OK) return 0;
  return make_layout(sh, gemm).total;
}

int moe_router_topk(const float* logits, int32_t T, int32_t E, int32_t k, float route_scale,
                    float top_p, int32_t score, const float* select_bias, int32_t n_group,
                    int32_t topk_group, int32_t* idx, float* w, moe_stream_t stream) {
  if (!logits || !idx || !w || T < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (!aligned(logits, 4) || !aligned(idx, 4) || !aligned(w, 4)) return MOE_ERR_INVALID_ARG;
  const int rc = check_router(score, select_bias, top_p, n_group, topk_group, E, k);
  if (rc != MOE_OK) return rc;
  if (E > 256 || k > 64) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_topk(
      logits, E, T, E, k,
      moe::RouterSpec{route_scale, top_p, score, select_bias, n_group, topk_group}, idx, w,
      moe::Launch{reinterpret_cast<hipStream_t>(stream)}));
}

int moe_pack_weights(moe_q4 src, int32_t E, int32_t N, int32_t K, int32_t format, moe_q4 dst,
                     moe_stream_t stream) {
  if (!plane_ok(src) || !plane_ok(dst)) return MOE_ERR_INVALID_ARG;
  if (E < 1 || N < 1 || K < 64 || N % 32 || K % 64) return MOE_ERR_INVALID_ARG;
  if (format != MOE_FORMAT_INT4 && format != MOE_FORMAT_MXFP4) return MOE_ERR_INVALID_ARG;
  const bool mx = format == MOE_FORMAT_MXFP4;
  const uintptr_t qb = (uintptr_t)E * N * (K / 2), sb = (uintptr_t)E * N * (K / 32) * (mx ? 1 : 2);
  auto overlap = [](const void* a, uintptr_t na, const void* b, uintptr_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
  };
  if (overlap(src.q, qb, dst.q, qb) || overlap(src.s, sb, dst.s, sb) ||
      overlap(src.q, qb, dst.s, sb) || overlap(src.s, sb, dst.q, qb))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_pack_weights(src.q, src.s, E, N, K, const_cast<uint8_t*>(dst.q),
                                             const_cast<void*>(dst.s),
                                             mx ? moe::kFmtMxfp4 : moe::kFmtInt4,
                                             moe::Launch{reinterpret_cast<hipStream_t>(stream)}));
}

size_t moe_permute_workspace_bytes(int32_t T, int32_t k, int32_t E) {
  if (T < 1 || k < 1 || E < 1 || E > 256 || (int64_t)T * k >= (int64_t)1 << 31) return 0;
  const int64_t slots = (int64_t)T * k;
  if (slots <= moe::kPermuteOneBlockMax) return 0;
  return sizeof(int32_t) * (size_t)moe::permute_scratch_words(slots, E);
}

int moe_permute(const int32_t* idx, int32_t T, int32_t k, int32_t E, int32_t* off,
                int32_t* sorted, int32_t* row_of, void* ws, size_t ws_bytes,
                moe_stream_t stream) {
  if (!idx || !off || !sorted || !row_of || T < 1 || k < 1 || E < 1) return MOE_ERR_INVALID_ARG;
  if (!aligned(idx, 4) || !aligned(off, 4) || !aligned(sorted, 4) || !aligned(row_of, 4) ||
      !aligned(ws, kAlign))
    return MOE_ERR_INVALID_ARG;
  if (E > 256) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * k >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  const size_t need = moe_permute_workspace_bytes(T, k, E);
  if (ws_bytes < need || (need && !ws)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_permute(idx, T, k, E, off, sorted, row_of, nullptr,
                                        need ? static_cast<int32_t*>(ws) : nullptr,
                                        moe::Launch{reinterpret_cast<hipStream_t>(stream)}));
}

int moe_expert_mlp(const moe_shape* sh, const uint16_t* x, const int32_t* off,
                   const int32_t* sorted, const float* w, moe_q4 gate, moe_q4 up, moe_q4 down,
                   float* y, void* ws, size_t ws_bytes, moe_stream_t stream) {
  int rc = check_shape(sh);
  if (rc != MOE_OK) return rc;
  if (!x || !off || !sorted || !w || !y || !ws) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(w, 4) || !aligned(ws, kAlign))
    return MOE_ERR_INVALID_ARG;
  if (!plane_ok(gate) || !plane_ok(up) || !plane_ok(down)) return MOE_ERR_INVALID_ARG;
  bool gemm = false;
  rc = pick_gemm(sh, &gemm);
  if (rc != MOE_OK) return rc;
  const Layout L = make_layout(sh, gemm);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (moe::launch_schedule_from_offsets(off, sh->E, (int64_t)sh->T * sh->k, at<int32_t>(ws, L.sched),
                                         moe::Launch{st}) != hipSuccess)
    return MOE_ERR_HIP;
  return run_mlp(sh, gemm, L, ws, x, off, sorted, w, gate, up, down, nullptr, nullptr, 0, y, st,
                 Stages{nullptr, st});
}

static int layer_impl(const moe_shape* sh, const uint16_t* x, const float* logits,
                      const float* w_router, moe_q4 gate, moe_q4 up, moe_q4 down,
                      const moe_q4* shared, const float* shared_gate, float* y, int32_t* idx_out,
                      float* w_out, float* logits_out, void* ws, size_t ws_bytes,
                      moe_stream_t stream, void* const* events, bool accumulate = false,
                      int32_t* stage_ran = nullptr) {
  int rc = check_shape(sh);
  if (rc != MOE_OK) return rc;
  if (!x || !y || !ws) return MOE_ERR_INVALID_ARG;
  if ((logits == nullptr) == (w_router == nullptr)) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, kAlign)) return MOE_ERR_INVALID_ARG;
  if (logits && !aligned(logits, 4)) return MOE_ERR_INVALID_ARG;
  if (w_router && !aligned(w_router, 16)) return MOE_ERR_INVALID_ARG;
  if ((idx_out && !aligned(idx_out, 4)) || (w_out && !aligned(w_out, 4)) ||
      (logits_out && !aligned(logits_out, 4)))
    return MOE_ERR_INVALID_ARG;
  if (!plane_ok(gate) || !plane_ok(up) || !plane_ok(down)) return MOE_ERR_INVALID_ARG;
  if (shared) {
    if (sh->SI < 64) return MOE_ERR_INVALID_ARG;
    for (int i = 0; i < 3; ++i)
      if (!plane_ok(shared[i])) return MOE_ERR_INVALID_ARG;
    if (shared_gate && !aligned(shared_gate, 16)) return MOE_ERR_INVALID_ARG;
  } else if (sh->SI != 0) {
    return MOE_ERR_INVALID_ARG;
  }
  bool gemm = false;
  rc = pick_gemm(sh, &gemm);
  if (rc != MOE_OK) return rc;
  const Layout L = make_layout(sh, gemm);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int T = sh->T, H = sh->H, E = sh->E, k = sh->k;
  const bool gated = shared && shared_gate;
  const Stages sg{events, st, stage_ran};
  if (!sg.skip(MOE_STAGE_START)) return MOE_ERR_HIP;

  // 1. logits (and the shared gate logit as one more router row)
  const float* Lp = logits;
  int ldL = E;
  const float* gate_logit = nullptr;
  int gate_ld = 1;
  if (w_router) {
    float* Lw = at<float>(ws, L.logits);
    const int ld = gated ? E + 1 : E;
    if (moe::launch_router_logits(x, w_router, gated ? shared_gate : nullptr, T, H, E, Lw, ld,
                                  gemm ? at<uint16_t>(ws, L.x16) : nullptr,
                                  sg.at(MOE_STAGE_LOGITS)) != hipSuccess)
      return MOE_ERR_HIP;
    Lp = Lw;
    ldL = ld;
    if (gated) {
      gate_logit = Lw + E;
      gate_ld = ld;
    }
  } else if (gated) {
    float* gl = at<float>(ws, L.gate);
    if (moe::launch_router_logits(x, nullptr, shared_gate, T, H, 0, gl, 1,
                                  gemm ? at<uint16_t>(ws, L.x16) : nullptr,
                                  sg.at(MOE_STAGE_LOGITS)) != hipSuccess)
      return MOE_ERR_HIP;
    gate_logit = gl;
    gate_ld = 1;
  } else if (!sg.skip(MOE_STAGE_LOGITS)) {
    return MOE_ERR_HIP;
  }
  if (logits_out) {
    if (hipMemcpy2DAsync(logits_out, sizeof(float) * E, Lp, sizeof(float) * ldL,
                         sizeof(float) * E, T, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return MOE_ERR_HIP;
  }
  // 2.-3. top-k + weights, permutation + schedule: folded into the gate/up
  // GEMV for a handful of tokens, one fused workgroup for decode-sized
  // batches, separate kernels beyond.
  int32_t* idx = idx_out ? idx_out : at<int32_t>(ws, L.idx);
  float* w = w_out ? w_out : at<float>(ws, L.w);
  int32_t* off = at<int32_t>(ws, L.off);
  int32_t* sorted = at<int32_t>(ws, L.sorted);
  const bool fold = !gemm && T <= moe::kFusedRouteMaxT && T * k <= moe::kFusedRouteMaxSlots;
  moe::RouteArgs ra{Lp, ldL, E, T, router_spec(sh), idx, w, off, sorted,
                    at<int32_t>(ws, L.row_of), at<int32_t>(ws, L.sched)};
  if (fold) {
    if (!sg.skip(MOE_STAGE_TOPK) || !sg.skip(MOE_STAGE_PERMUTE)) return MOE_ERR_HIP;
  } else if ((int64_t)T * k <= moe::kRouteMaxSlots && T <= moe::kRouteMaxT) {
    if (moe::launch_route(Lp, ldL, T, E, k, router_spec(sh), idx, w, off, sorted,
                          at<int32_t>(ws, L.row_of), at<int32_t>(ws, L.sched),
                          sg.at(MOE_STAGE_TOPK)) != hipSuccess ||
        !sg.skip(MOE_STAGE_PERMUTE))
      return MOE_ERR_HIP;
  } else {
    if (moe::launch_topk(Lp, ldL, T, E, k, router_spec(sh), idx, w,
                         sg.at(MOE_STAGE_TOPK)) != hipSuccess)
      return MOE_ERR_HIP;
    if (moe::launch_permute(idx, T, k, E, off, sorted, at<int32_t>(ws, L.row_of),
                            at<int32_t>(ws, L.sched), at<int32_t>(ws, L.pscratch),
                            sg.at(MOE_STAGE_PERMUTE)) != hipSuccess)
      return MOE_ERR_HIP;
  }

  // 4.-5. expert MLPs with the fused combine
  const bool x16_ready = gemm && (w_router || gated);
  return run_mlp(sh, gemm, L, ws, x, off, sorted, w, gate, up, down, shared, gate_logit, gate_ld,
                 y, st, sg, fold ? &ra : nullptr, x16_ready, accumulate);
}

int moe_layer(const moe_shape* sh, const uint16_t* x, const float* logits,
              const float* w_router, moe_q4 gate, moe_q4 up, moe_q4 down, const moe_q4* shared,
              const float* shared_gate, float* y, int32_t* idx_out, float* w_out,
              float* logits_out, void* ws, size_t ws_bytes, moe_stream_t stream) {
  return layer_impl(sh, x, logits, w_router, gate, up, down, shared, shared_gate, y, idx_out,
                    w_out, logits_out, ws, ws_bytes, stream, nullptr);
}

int moe_layer_static(const moe_shape* sh, const uint16_t* x, const float* logits,
                     const float* w_router, moe_q4 gate, moe_q4 up, moe_q4 down,
                     const moe_q4* shared, const float* shared_gate, float* y, int32_t* idx_out,
                     float* w_out, float* logits_out, moe_stream_t stream) {
  // A shape the layer does not serve needs 0 bytes; layer_impl then returns
  // its own error before anything is enqueued.
  const size_t need = moe_workspace_bytes(sh);
  if (need > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  const int rc = static_scratch(&ws);
  if (rc != MOE_OK) return rc;
  return layer_impl(sh, x, logits, w_router, gate, up, down, shared, shared_gate, y, idx_out,
                    w_out, logits_out, ws, (size_t)MOE_STATIC_SCRATCH_BYTES, stream, nullptr);
}

int moe_layer_residual_rmsnorm(const moe_shape* sh, const uint16_t* x, const float* logits,
                               const float* w_router, moe_q4 gate, moe_q4 up, moe_q4 down,
                               const moe_q4* shared, const float* shared_gate, float* residual,
                               const float* norm_w, float eps, uint16_t* x_next,
                               const float* next_w_router, int32_t next_E, float* next_logits,
                               int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes,
                               moe_stream_t stream) {
  if (!residual || !norm_w || !x_next || !aligned(residual, 16) || !aligned(norm_w, 16) ||
      !aligned(x_next, 16) || !(eps >= 0.0f))
    return MOE_ERR_INVALID_ARG;
  if ((next_w_router == nullptr) != (next_logits == nullptr)) return MOE_ERR_INVALID_ARG;
  if (next_w_router &&
      (next_E < 1 || !aligned(next_w_router, 16) || !aligned(next_logits, 4)))
    return MOE_ERR_INVALID_ARG;
  if (sh && sh->H % 4) return MOE_ERR_UNSUPPORTED;
  const int rc = layer_impl(sh, x, logits, w_router, gate, up, down, shared, shared_gate,
                            residual, idx_out, w_out, nullptr, ws, ws_bytes, stream, nullptr,
                            true);
  if (rc != MOE_OK) return rc;
  const moe::Launch L{reinterpret_cast<hipStream_t>(stream)};
  if (next_w_router)
    return hip_status(moe::launch_rmsnorm_router(residual, norm_w, sh->T, sh->H, eps, x_next,
                                                 next_w_router, next_E, next_logits, L));
  return hip_status(moe::launch_rmsnorm(residual, norm_w, sh->T, sh->H, eps, x_next, L));
}

int moe_layer_profiled(const moe_shape* sh, const uint16_t* x, const float* logits,
                       const float* w_router, moe_q4 gate, moe_q4 up, moe_q4 down,
                       const moe_q4* shared, const float* shared_gate, float* y,
                       int32_t* idx_out, float* w_out, float* logits_out, void* ws,
                       size_t ws_bytes, moe_stream_t stream, void* const* events,
                       int32_t n_events, int32_t* stage_ran) {
  if (!events || n_events < 2 * MOE_STAGE_COUNT) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < 2 * MOE_STAGE_COUNT; ++i)
    if (!events[i]) return MOE_ERR_INVALID_ARG;
  return layer_impl(sh, x, logits, w_router, gate, up, down, shared, shared_gate, y, idx_out,
                    w_out, logits_out, ws, ws_bytes, stream, events, false, stage_ran);
}



int moe_debug_read_probe(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink,
                         moe_stream_t stream) {
  if (!src || !sink || bytes < 16 || bytes % 16 || !aligned(src, 16) || !aligned(sink, 4) ||
      workgroups < 1 || workgroups > (1 << 20))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_read_probe(src, (int64_t)bytes, workgroups, sink,
                                           moe::Launch{reinterpret_cast<hipStream_t>(stream)}));
}

int moe_debug_dequant_int4(moe_q4 plane, int32_t N, int32_t K, int32_t mode, float* out,
                           moe_stream_t stream) {
  if (!plane_ok(plane) || !out || N < 1 || K < 32 || K % 32 || mode < 0 || mode > 3)
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_debug_dequant(plane.q, plane.s, N, K, mode, out,
                                              moe::Launch{reinterpret_cast<hipStream_t>(stream)}));
}

int moe_debug_dequant_mxfp4(moe_q4 plane, int32_t N, int32_t K, int32_t mode, float* out,
                            moe_stream_t stream) {
  if (!plane_ok(plane) || !out || N < 1 || K < 32 || K % 32 || mode < 0 || mode > 2)
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_debug_dequant(plane.q, plane.s, N, K, moe::kDebugMx4Gemv + mode,
                                              out,
                                              moe::Launch{reinterpret_cast<hipStream_t>(stream)}));
}

}  // extern "C"
