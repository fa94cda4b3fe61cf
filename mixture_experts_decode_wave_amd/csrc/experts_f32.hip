// Expert-pass kernels for f32 weights (one file per format so they build in parallel).
#include "experts_impl.h"

namespace moe {
hipError_t launch_expert_f32(bool mfma, int nmat, int tr, const GemvArgs &a, int grid,
                          hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return launch_expert_fmt<FMT_F32>(mfma, nmat, tr, a, grid, s, e0, e1);
}
hipError_t launch_down_blend1_f32(const Down1Args &a, int lds_bytes, hipStream_t s,
                                 hipEvent_t e0, hipEvent_t e1) {
  return launch_down_blend1_fmt<FMT_F32>(a, lds_bytes, s, e0, e1);
}
}  // namespace moe
