// Explicit instantiations of the single-launch layer kernel (fused_kernel.h),
// grouped in five units.  One unit's kernels take about a minute to compile,
// so the library build compiles this file once per unit, with
// -DMOE_FUSED_UNIT=0..4, and the units build in parallel; without the macro
// the file holds every unit.
//   0: MXFP4 (the VALU down paths and the matrix-core MFMA16 down path)
//   1: MXFP4 with the matrix-core down path and the RMS normalisation of the
//      residual stream in the kernel (the steps of a layer stack)
//   2: Q2_K
//   3: INT4 group-32
//   4: per-family precision: gate and up in MXFP4 or INT4 group-32, the down
//      projection in Q2_K
#include "fused_kernel.h"

#if !defined(MOE_FUSED_UNIT)
#define MOE_UNIT(n) 1
#elif MOE_FUSED_UNIT >= 0 && MOE_FUSED_UNIT <= 4
#define MOE_UNIT(n) (MOE_FUSED_UNIT == (n))
#else
#error "MOE_FUSED_UNIT must be 0..4"
#endif

namespace moe {
namespace fused {

#if MOE_UNIT(0)
hipError_t launch_mx(const FusedArgs& a, int grid, int gu_units, int dn_units, int ups, hipStream_t s) {
  return launch_fused_ups<MxFmt>(a, grid, gu_units, dn_units, ups, s);
}

hipError_t launch_mx_mfma(const FusedArgs& a, int grid, int gu_units, int ups, hipStream_t s) {
  return launch_fused_mfma<false>(a, grid, gu_units, ups, s);
}
#endif

#if MOE_UNIT(1)
hipError_t launch_mx_mfma_norm(const FusedArgs& a, int grid, int gu_units, int ups, hipStream_t s) {
  return launch_fused_mfma<true>(a, grid, gu_units, ups, s);
}
#endif

#if MOE_UNIT(2)
hipError_t launch_q2k(const FusedArgs& a, int grid, int gu_units, int dn_units, int ups, hipStream_t s) {
  return launch_fused_ups<Q2kFmt>(a, grid, gu_units, dn_units, ups, s);
}
#endif

#if MOE_UNIT(3)
hipError_t launch_int4(const FusedArgs& a, int grid, int gu_units, int dn_units, int ups, hipStream_t s) {
  return launch_fused_ups<Int4Fmt>(a, grid, gu_units, dn_units, ups, s);
}
#endif

#if MOE_UNIT(4)
hipError_t launch_mx_q2k(const FusedArgs& a, int grid, int gu_units, int dn_units, int ups, hipStream_t s) {
  return launch_fused_ups<MxFmt, Q2kFmt>(a, grid, gu_units, dn_units, ups, s);
}

hipError_t launch_int4_q2k(const FusedArgs& a, int grid, int gu_units, int dn_units, int ups, hipStream_t s) {
  return launch_fused_ups<Int4Fmt, Q2kFmt>(a, grid, gu_units, dn_units, ups, s);
}
#endif

}  // namespace fused
}  // namespace moe
