// jas_kernels_bf16.hip -- the bf16 instances of the row-softmax kernels.

#include "jas_kernels.h"

namespace jas {

hipError_t launch_fwd_bf16(const FwdArgs &a, const Geometry &g, hipStream_t st) {
  return fwd_dt<1>(a, g, st);
}

hipError_t launch_bwd_bf16(const BwdArgs &a, const Geometry &g, hipStream_t st) {
  return bwd_dt<1>(a, g, st);
}

}  // namespace jas
