// fused_bf16.hip -- one workgroup per (batch, head) slice for short sequences.
#include "device_common.h"
#include "kernels.h"

namespace aa {

bool fused_supported(const Geometry&, FusedPlan*) { return false; }

hipError_t launch_fused_bf16(const Geometry&, const FusedPlan&, const void*, const void*,
                             const void*, void*, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace aa
