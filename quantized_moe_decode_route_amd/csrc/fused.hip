// Host side of the single-launch layer: shape checks, XCD placement probe
// and the dispatch to the per-format kernels (fused_kernel.h).
#include "fused_kernel.h"

#include <cstdlib>

namespace moe {
using fused::FusedArgs;
using fused::kW;
using fused::kMaxNX;
using fused::kLdsBytes;
using fused::xcc_id;
namespace {

// Records each workgroup's XCD.  Its LDS footprint matches the layer
// kernel's, so the placement is the same one-workgroup-per-CU placement.
__global__ __launch_bounds__(kW * kWave, 1) void xcc_map_kernel(uint32_t* out) {
  extern __shared__ uint32_t lds_footprint[];  // sized at launch like the layer kernel's LDS
  if (threadIdx.x == 0) {
    lds_footprint[0] = xcc_id();
    out[blockIdx.x] = lds_footprint[0];
  }
}

// Per device: 1 when the probe saw workgroup b on XCD b % nx.
int& rr_slot(int dev) {
  static int rr[64] = {0};
  return rr[dev];
}

}  // namespace

FusedShape fused_shape(int fmt, int dfmt, int B, int k, int D, int F, int grid, int nx, int down_layout) {
  FusedShape sh{};
  sh.ok = false;
  sh.mfma = down_layout == MOE_LAYOUT_MFMA16;
  if (sh.mfma && (fmt != MOE_FMT_MXFP4 || dfmt != MOE_FMT_MXFP4)) return sh;
  // mixed formats: gate/up in MXFP4 or INT4 with a Q2_K down projection
  if (dfmt != fmt && !(dfmt == MOE_FMT_Q2K && (fmt == MOE_FMT_MXFP4 || fmt == MOE_FMT_INT4G32))) return sh;
  if (grid <= 0 || nx <= 0 || nx > kMaxNX || grid % nx) return sh;
  const int uwg = fmt == MOE_FMT_Q2K ? 64 : 32;   // unit width of gate/up (along d_model)
  const int uw = dfmt == MOE_FMT_Q2K ? 64 : 32;   // unit width of down (along d_ff)
  const int gx = grid / nx;
  if (F % (nx * uw)) return sh;  // every XCD's d_ff slice is whole units
  const int ups = F / nx / uw;
  if (ups != 1 && ups != 2 && ups != 4 && ups != 8 && ups != 16) return sh;
  sh.gu_units = D / uwg;
  if (D % uwg || sh.gu_units > 2 * kWave) return sh;
  const int rpwd = (D + gx - 1) / gx;
  const int rpv = (rpwd + kW - 1) / kW;
  sh.dn_units = rpv * ups;
  if (sh.dn_units > 2 * kWave) return sh;
  sh.ups = ups;
  // LDS: activations during gate/up, then h slices and row partials.
  const size_t staged = fmt == MOE_FMT_Q2K ? 4 * Q2kFmt::kXDw : fmt == MOE_FMT_INT4G32 ? 4 * Int4Fmt::kXDw : 4 * MxFmt::kXDw;
  const size_t act = (size_t)B * (D / uwg) * staged;
  size_t down = (size_t)B * k * ups * (uw + 4) * 4 + (size_t)B * k * rpwd * 4;
  if (sh.mfma) {
    // one 16-row tile per wave, at most two 128-column k-steps per XCD
    // slice; the B operands (kHTerms E4M3 terms of 128 values per k-step and
    // slot, plus the zero slot) and row partials replace the activations
    if (rpv > 16 || ups > 8) return sh;
    const size_t S = (size_t)B * k, dnk = (ups + 3) / 4;
    auto up16 = [](size_t v) { return (v + 15) & ~(size_t)15; };
    down = (S + 1) * dnk * 128 * fused::kHTerms + up16((S + 1) * 4 * dnk) + S * rpwd * 4;
  }
  if (act > (size_t)kLdsBytes || down > (size_t)kLdsBytes) return sh;
  sh.ok = true;
  return sh;
}

int fused_grid_size() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static int cached[64] = {0};
  if (dev >= 0 && dev < 64 && cached[dev]) return cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) cached[dev] = cus;
  return cus;
}

namespace {
int& xcd_count_slot(int dev) {
  static int nx[64] = {0};  // per device: 0 unknown, -1 unusable, else the XCD count
  return nx[dev];
}
}  // namespace

int xcd_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  return xcd_count_slot(dev);
}

int probe_xcd_count(uint32_t* scratch, int grid, hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  int& nx = xcd_count_slot(dev);
  if (nx) return nx;
  if (grid <= 0 || grid > 4096) return nx = -1;
  hipLaunchKernelGGL(xcc_map_kernel, dim3(grid), dim3(kW * kWave), kLdsBytes + 8 * 1024, s, scratch);
  uint32_t host[4096];
  if (hipMemcpyAsync(host, scratch, sizeof(uint32_t) * grid, hipMemcpyDeviceToHost, s) != hipSuccess) return -1;
  if (hipStreamSynchronize(s) != hipSuccess) return -1;
  int count[kMaxNX] = {0};
  int n = 0;
  for (int b = 0; b < grid; ++b) {
    const uint32_t x = host[b];
    if (x >= (uint32_t)kMaxNX) return nx = -1;
    ++count[x];
    if ((int)x + 1 > n) n = (int)x + 1;
  }
  // Every XCD must hold the same number of workgroups.
  for (int x = 0; x < n; ++x)
    if (count[x] * n != grid) return nx = -1;
  // Workgroup indices inside an XCD from the block index when the placement
  // is round-robin (workgroup b on XCD b % n), unless MOE_XCD_INDEX_ATOMIC is
  // set; otherwise the kernel takes them from an L2 atomic counter.
  bool rr = true;
  for (int b = 0; b < grid; ++b) rr = rr && (int)host[b] == b % n;
  const char* env = std::getenv("MOE_XCD_INDEX_ATOMIC");
  rr_slot(dev) = rr && !(env && env[0] && env[0] != '0');
  return nx = n;
}

hipError_t launch_fused_layer(int fmt, int dfmt, const float* router_w, const uint16_t* x, const float* hn, double eps,
                              const WeightRef& gate, const WeightRef& up, const WeightRef& down, int E, int D, int Fd,
                              int k, int B, uint8_t* ws, const WsLayout& L, float* y, const float* residual,
                              int32_t* idx_out, float* gw_out, uint64_t* trace, hipStream_t s,
                              const HashRoute& hr, const float* next_router) {
  static_assert(kW == kRmsWaves, "the in-kernel norm sums over the norm kernel's eight waves");
  if (hn && (B != 1 || D > kFusedNormMaxD || D % 8 || hn == y)) return hipErrorInvalidValue;
  FusedArgs a;
  a.router_w = router_w;
  a.x = x;
  a.hn = hn;
  a.eps = eps;
  a.hr = hr;
  a.next_router = next_router;
  a.gate = gate;
  a.up = up;
  a.down = down;
  a.ws = ws;
  a.L = L;
  a.y = y;
  a.residual = residual;
  a.idx_out = idx_out;
  a.gw_out = gw_out;
  a.trace = trace;
  a.E = E;
  a.D = D;
  a.Fd = Fd;
  a.k = k;
  a.B = B;
  a.nx = xcd_count();
  {
    int dev = 0;
    a.rr_mode = hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64 ? rr_slot(dev) : 0;
  }
  const int grid = fused_grid_size();
  const FusedShape sh = fused_shape(fmt, dfmt, B, k, D, Fd, grid, a.nx, down.layout);
  if (!sh.ok) return hipErrorInvalidValue;
  if (dfmt != fmt) {
    if (hn) return hipErrorInvalidValue;
    return fmt == MOE_FMT_MXFP4 ? fused::launch_mx_q2k(a, grid, sh.gu_units, sh.dn_units, sh.ups, s)
                                : fused::launch_int4_q2k(a, grid, sh.gu_units, sh.dn_units, sh.ups, s);
  }
  if (sh.mfma) {
    return hn ? fused::launch_mx_mfma_norm(a, grid, sh.gu_units, sh.ups, s)
              : fused::launch_mx_mfma(a, grid, sh.gu_units, sh.ups, s);
  }
  if (hn) return hipErrorInvalidValue;  // the in-kernel norm is built for the matrix-core path only
  switch (fmt) {
    case MOE_FMT_MXFP4: return fused::launch_mx(a, grid, sh.gu_units, sh.dn_units, sh.ups, s);
    case MOE_FMT_Q2K: return fused::launch_q2k(a, grid, sh.gu_units, sh.dn_units, sh.ups, s);
    case MOE_FMT_INT4G32: return fused::launch_int4(a, grid, sh.gu_units, sh.dn_units, sh.ups, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
