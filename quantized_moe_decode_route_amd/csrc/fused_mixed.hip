// Single-launch layer kernels with per-family precision: gate and up in
// MXFP4 or INT4 group-32, the down projection in Q2_K.
#include "fused_kernel.h"

namespace moe {
namespace fused {

hipError_t launch_mx_q2k(const FusedArgs& a, int grid, int gu_units, int dn_units, int ups, hipStream_t s) {
  return launch_fused_ups<MxFmt, Q2kFmt>(a, grid, gu_units, dn_units, ups, s);
}

hipError_t launch_int4_q2k(const FusedArgs& a, int grid, int gu_units, int dn_units, int ups, hipStream_t s) {
  return launch_fused_ups<Int4Fmt, Q2kFmt>(a, grid, gu_units, dn_units, ups, s);
}

}  // namespace fused
}  // namespace moe
