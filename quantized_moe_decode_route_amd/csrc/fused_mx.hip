// Single-launch layer kernels for one weight format (the kernel template is
// in fused_kernel.h; one file per format keeps the builds parallel).
#include "fused_kernel.h"

namespace moe {
namespace fused {

hipError_t launch_mx(const FusedArgs& a, int grid, int gu_units, int dn_units, int ups, hipStream_t s) {
  return launch_fused_ups<MxFmt>(a, grid, gu_units, dn_units, ups, s);
}

hipError_t launch_mx_mfma(const FusedArgs& a, int grid, int gu_units, int ups, hipStream_t s) {
  return launch_fused_mfma<false>(a, grid, gu_units, ups, s);
}

}  // namespace fused
}  // namespace moe
