// jas_kernels_f32.hip -- the fp32 instances of the row-softmax kernels.

#include "jas_kernels.h"

namespace jas {

hipError_t launch_fwd_f32(const FwdArgs &a, const Geometry &g, hipStream_t st) {
  return fwd_dt<0>(a, g, st);
}

hipError_t launch_bwd_f32(const BwdArgs &a, const Geometry &g, hipStream_t st) {
  return bwd_dt<0>(a, g, st);
}

}  // namespace jas
