// Streaming GEMV, MXFP4 instantiations of the kernels in gemv_impl.h (a
// translation unit of its own so the two formats compile in parallel).
#include "gemv_impl.h"

namespace moe {

hipError_t launch_gemv_gate_up_mxfp4(const Buckets& b, int max_buckets, const uint16_t* x, int H,
                                     int I, const uint8_t* gq, const void* gs, const uint8_t* uq,
                                     const void* us, uint16_t* h, float* y_zero, int64_t y_elems,
                                     const Launch& L, const RouteArgs* route) {
  return gemv_gate_up_launch<kFmtMxfp4>(b, max_buckets, x, H, I, gq, gs, uq, us, h, y_zero,
                                        y_elems, L, route);
}

hipError_t launch_gemv_down_mxfp4(const Buckets& b, int max_buckets, const uint16_t* h, int H,
                                  int I, const uint8_t* dq, const void* ds, const float* w,
                                  const float* gate_logit, int gate_ld, float* y, const Launch& L) {
  return gemv_down_launch<kFmtMxfp4>(b, max_buckets, h, H, I, dq, ds, w, gate_logit, gate_ld, y,
                                     L);
}

}  // namespace moe
