// Single-launch layer kernels for one weight format (the kernel template is
// in fused_kernel.h; one file per format keeps the builds parallel).
#include "fused_kernel.h"

namespace moe {
namespace fused {

hipError_t launch_q2k(const FusedArgs& a, int grid, int gu_units, int dn_units, int ups, hipStream_t s) {
  return launch_fused_ups<Q2kFmt>(a, grid, gu_units, dn_units, ups, s);
}

}  // namespace fused
}  // namespace moe
