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

// fp64 -> bfloat16 bits, round to nearest even, without double rounding:
// first to fp32 with round-to-odd (24 >= 8 + 2 bits), then fp32 -> bf16 RNE.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double v) {
  float f = (float)v;
  const double back = (double)f;
  if (back != v && !__builtin_isnan(v)) {
    uint32_t u = __float_as_uint(f);
    if (__builtin_fabs(back) > __builtin_fabs(v)) u -= 1u;  // step toward zero
    u |= 1u;
    f = __uint_as_float(u);
  }
  return f32_to_bf16_rne(f);
}

// One workgroup per token: x = bf16_rne(h / sqrt(mean(h^2) + eps)) in fp64.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ h, int D, double eps,
                                                      uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const float* row = h + (int64_t)t * D;
  double ss = 0.0;
  for (int i = threadIdx.x; i < D; i += blockDim.x) {
    const double v = row[i];
    ss = __builtin_fma(v, v, ss);
  }
  ss = wave_sum_f64(ss);
  __shared__ double s_part[4];
  if (lane_id() == 0) s_part[threadIdx.x / kWave] = ss;
  __syncthreads();
  const double tot = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
  const double denom = sqrt(tot / D + eps);
  for (int i = threadIdx.x; i < D; i += blockDim.x)
    out[(int64_t)t * D + i] = (uint16_t)f64_to_bf16_rne((double)row[i] / denom);
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
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(B), dim3(256), 0, s, h, D, eps, out);
  return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t s) {
  hipLaunchKernelGGL(zero_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace moe
