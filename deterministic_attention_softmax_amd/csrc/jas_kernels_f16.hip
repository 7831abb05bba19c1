// jas_kernels_f16.hip -- the fp16 (IEEE binary16) instances of the
// row-softmax kernels.

#include "jas_kernels.h"

namespace jas {

hipError_t launch_fwd_f16(const FwdArgs &a, const Geometry &g, hipStream_t st) {
  return fwd_dt<2>(a, g, st);
}

hipError_t launch_bwd_f16(const BwdArgs &a, const Geometry &g, hipStream_t st) {
  return bwd_dt<2>(a, g, st);
}

}  // namespace jas
