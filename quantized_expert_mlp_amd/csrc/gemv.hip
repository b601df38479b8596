// Streaming GEMV entry points: the int4 instantiations of the kernels in
// gemv_impl.h, and the dispatch by weight format.
#include "gemv_impl.h"

namespace moe {

bool gemv_supported(int K) { return K % 32 == 0 && K / 32 <= 4 * 64; }

hipError_t launch_gemv_gate_up(const Buckets& b, int max_buckets, const uint16_t* x, int H,
                               int I, const uint8_t* gq, const void* gs, const uint8_t* uq,
                               const void* us, uint16_t* h, float* y_zero, int64_t y_elems,
                               int fmt, const Launch& L, const RouteArgs* route) {
  if (fmt == kFmtMxfp4)
    return launch_gemv_gate_up_mxfp4(b, max_buckets, x, H, I, gq, gs, uq, us, h, y_zero, y_elems,
                                     L, route);
  return gemv_gate_up_launch<kFmtInt4>(b, max_buckets, x, H, I, gq, gs, uq, us, h, y_zero,
                                       y_elems, L, route);
}

hipError_t launch_gemv_down(const Buckets& b, int max_buckets, const uint16_t* h, int H, int I,
                            const uint8_t* dq, const void* ds, const float* w,
                            const float* gate_logit, int gate_ld, float* y, int fmt,
                            const Launch& L) {
  if (fmt == kFmtMxfp4)
    return launch_gemv_down_mxfp4(b, max_buckets, h, H, I, dq, ds, w, gate_logit, gate_ld, y, L);
  return gemv_down_launch<kFmtInt4>(b, max_buckets, h, H, I, dq, ds, w, gate_logit, gate_ld, y,
                                    L);
}

}  // namespace moe
