// Small layer kernels: rank-ordered weighted combine of the expert outputs
// (optionally onto a residual), the RMSNorm that feeds each stacked layer,
// and the workspace counter reset.
#include "moe_internal.h"

namespace moe {
namespace {

// y[t][n] = residual[t][n] + sum_j gw[t][j] * yp[t][j][n], j ascending.
// One thread per 4 consecutive outputs.
__global__ __launch_bounds__(256) void combine_kernel(int D, int B, int k, const uint8_t* __restrict__ ws,
                                                      WsLayout L, float* y, const float* residual) {
  const int64_t i4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n4 = (int64_t)B * D / 4;
  if (i4 >= n4) return;
  const int t = (int)(i4 * 4 / D);
  const int n = (int)(i4 * 4 - (int64_t)t * D);
  const float* gw = reinterpret_cast<const float*>(ws + L.gw) + t * k;
  const float* yp = reinterpret_cast<const float*>(ws + L.yp) + (int64_t)t * k * D + n;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float g = gw[j];
    const float4 v = *reinterpret_cast<const float4*>(yp + (int64_t)j * D);
    acc.x = __builtin_fmaf(g, v.x, acc.x);
    acc.y = __builtin_fmaf(g, v.y, acc.y);
    acc.z = __builtin_fmaf(g, v.z, acc.z);
    acc.w = __builtin_fmaf(g, v.w, acc.w);
  }
  if (residual) {
    const float4 r = *reinterpret_cast<const float4*>(residual + (int64_t)t * D + n);
    acc.x += r.x;
    acc.y += r.y;
    acc.z += r.z;
    acc.w += r.w;
  }
  *reinterpret_cast<float4*>(y + (int64_t)t * D + n) = acc;
}

// One workgroup per token: x = bf16_rne(h / sqrt(mean(h^2) + eps)) in fp64,
// the sum of squares in the chunk order of rms_total.  Rows of at most 4096
// elements (a multiple of 8, 16-byte aligned) take one chunk per thread with
// both of its loads issued at once; other rows walk their chunks in the same
// order element by element.
__global__ __launch_bounds__(kRmsThreads) void rmsnorm_kernel(const float* __restrict__ h, int D, double eps,
                                                              uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const float* row = h + (int64_t)t * D;
  uint16_t* xo = out + (int64_t)t * D;
  const int i = threadIdx.x;
  __shared__ double s_part[kRmsWaves];
  const bool vec = D % 8 == 0 && D <= 8 * kRmsThreads && (((uintptr_t)h | (uintptr_t)out) & 15u) == 0;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
  double ss = 0.0;
  if (vec) {
    if (8 * i < D) {
      a = *reinterpret_cast<const float4*>(row + 8 * i);
      b = *reinterpret_cast<const float4*>(row + 8 * i + 4);
      ss = rms_squares8(a, b, 0.0);
    }
  } else {
    for (int c = i; 8 * c < D; c += kRmsThreads)
      for (int j = 8 * c; j < min(8 * c + 8, D); ++j) {
        const double v = row[j];
        ss = __builtin_fma(v, v, ss);
      }
  }
  ss = wave_sum_dpp_f64(ss);
  if (lane_id() == kWave - 1) s_part[i / kWave] = ss;
  __syncthreads();
  const RmsScale sc = rms_scale(rms_total(s_part), D, eps);
  if (vec) {
    if (8 * i < D) {
      bool near = !sc.fast;
      uint4 x = rms_x8_fast(a, b, sc.r, near);
      if (near) x = rms_x8_exact(a, b, sc.denom);
      *reinterpret_cast<uint4*>(xo + 8 * i) = x;
    }
  } else {
    // element by element (the same values: the fast form only ever returns
    // the correctly rounded quotient)
    for (int c = i; 8 * c < D; c += kRmsThreads)
      for (int j = 8 * c; j < min(8 * c + 8, D); ++j) xo[j] = (uint16_t)f64_to_bf16_rne((double)row[j] / sc.denom);
  }
}

__global__ void zero_u32_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t launch_combine(int D, int B, int k, const uint8_t* ws, const WsLayout& L, float* y, const float* residual,
                          hipStream_t s) {
  const int64_t n4 = (int64_t)B * D / 4;
  dim3 grid((unsigned)((n4 + 255) / 256));
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, D, B, k, ws, L, y, residual);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bf16(const float* h, int B, int D, double eps, uint16_t* out, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(B), dim3(kRmsThreads), 0, s, h, D, eps, out);
  return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t s) {
  hipLaunchKernelGGL(zero_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace moe
