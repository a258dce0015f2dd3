// Single-launch MXFP4 layer kernels (matrix-core down projection) that
// RMS-normalise the residual stream themselves: the steps of a layer stack.
#include "fused_kernel.h"

namespace moe {
namespace fused {

hipError_t launch_mx_mfma_norm(const FusedArgs& a, int grid, int gu_units, int ups, hipStream_t s) {
  return launch_fused_mfma<true>(a, grid, gu_units, ups, s);
}

}  // namespace fused
}  // namespace moe
