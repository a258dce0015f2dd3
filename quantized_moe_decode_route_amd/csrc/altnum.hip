// Alternative numerics for the MXFP4 matvec, measured against the main path
// ("ds4.c study notes", glossary page "quantization"):
//  * "MXFP4's ROCm native kernel": activations quantized to Q8_K, weights'
//    codes expanded to int8 with v_perm and dotted as integers (v_dot4);
//  * "Metal's MXFP4 -> half lookup table": every weight decoded by one
//    indexed load from a 256 x 16 table of exactly rounded binary16 products.
// The main path instead widens codes with gfx950's FP4 conversion and keeps
// the activations exact; these two exist to compare numerics and VALU cost.
#include <hip/hip_fp16.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kAltR = 2;  // rows per wave

__device__ __forceinline__ float wave_max_shfl(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// One workgroup per (256-activation block, token): d = max|x| / 127 and
// q = clamp(rint(x / d), -127, 127), in fp32 (IEEE division, ties to even).
__global__ __launch_bounds__(256) void q8k_quantize_kernel(const float* __restrict__ x, int K, int8_t* __restrict__ q,
                                                           float* __restrict__ d) {
  __shared__ float s_max[4];
  const int b = blockIdx.x, t = blockIdx.y, i = threadIdx.x;
  const int64_t o = (int64_t)t * K + 256 * b + i;
  const float v = x[o];
  const float m = wave_max_shfl(fabsf(v));
  if ((i & (kWave - 1)) == 0) s_max[i / kWave] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float db = amax / 127.0f;
  float r = db > 0.0f ? rintf(v / db) : 0.0f;
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  q[o] = (int8_t)(int)r;
  if (i == 0) d[(int64_t)t * (K / 256) + b] = db;
}

// Eight E2M1 codes (one code dword: byte j holds element 2j in its high
// nibble) -> twice their values as int8, in element order: lo = elements
// 0..3, hi = elements 4..7.  v_perm looks the magnitudes up in a byte table
// (codes 0..7 -> 0,1,2,3,4,6,8,12 and their negatives), bit 3 picks the sign.
__device__ __forceinline__ void codes_to_i8(uint32_t c, uint32_t& lo, uint32_t& hi) {
  const uint32_t L = c & 0x0F0F0F0Fu, H = (c >> 4) & 0x0F0F0F0Fu;
  const uint32_t a[2] = {__builtin_amdgcn_perm(L, H, 0x05010400u), __builtin_amdgcn_perm(L, H, 0x07030602u)};
  uint32_t r[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t sel = a[k] & 0x07070707u;
    const uint32_t pos = __builtin_amdgcn_perm(0x0C080604u, 0x03020100u, sel);
    const uint32_t neg = __builtin_amdgcn_perm(0xF4F8FAFCu, 0xFDFEFF00u, sel);
    const uint32_t mask = ((a[k] >> 3) & 0x01010101u) * 0xFFu;
    r[k] = (neg & mask) | (pos & ~mask);
  }
  lo = r[0];
  hi = r[1];
}

// y[t][n] = sum over blocks j of 2^(e - 128) * d[t][j/8] * (integer dot of
// the block's doubled codes with q[t][32j..32j+31]).  Lane l takes blocks
// l, l+64, ...; each wave computes kAltR rows.
__global__ __launch_bounds__(256) void gemv_q8_kernel(const uint8_t* __restrict__ w, int N, int K,
                                                      const int8_t* __restrict__ q, const float* __restrict__ d, int B,
                                                      float* __restrict__ y) {
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int row0 = (blockIdx.x * 4 + wave) * kAltR;
  if (row0 >= N) return;
  const int U = K / 32;
  for (int t = 0; t < B; ++t) {
    float acc[kAltR];
#pragma unroll
    for (int r = 0; r < kAltR; ++r) acc[r] = 0.0f;
    for (int u = lane; u < U; u += kWave) {
      const uint4 x0 = *reinterpret_cast<const uint4*>(q + (int64_t)t * K + 32 * u);
      const uint4 x1 = *reinterpret_cast<const uint4*>(q + (int64_t)t * K + 32 * u + 16);
      const uint32_t xq[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      const float du = d[(int64_t)t * (K / 256) + u / 8];
#pragma unroll
      for (int r = 0; r < kAltR; ++r) {
        const uint8_t* row = w + (int64_t)min(row0 + r, N - 1) * U * 17;
        MxRaw raw;
        mx_load(row, 17u * u, raw);
        uint32_t e, c[4];
        mx_unpack(raw, e, c);
        int isum = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t lo, hi;
          codes_to_i8(c[k], lo, hi);
          isum = __builtin_amdgcn_sdot4((int)lo, (int)xq[2 * k], isum, false);
          isum = __builtin_amdgcn_sdot4((int)hi, (int)xq[2 * k + 1], isum, false);
        }
        acc[r] = __builtin_fmaf(ldexpf((float)isum, (int)e - 128), du, acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < kAltR; ++r) {
      const float s = wave_sum_dpp(acc[r]);  // the total lands in lane 63
      if (lane == kWave - 1 && row0 + r < N) y[(int64_t)t * N + row0 + r] = s;
    }
  }
}

// Entry [e][c] of the binary16 table: E2M1(c) * 2^(e - 127) is exact in fp32
// (from 2^-128 up; products past fp32's range are infinite, as they are in
// binary16), and the conversion to binary16 rounds it once to nearest-even.
// Row 255 (an infinite scale) is the quiet NaN.
__device__ __forceinline__ uint16_t half_entry(int e, int c) {
  if (e == 255) return 0x7E00u;
  const f32x2 p = MOE_FP4X2((uint32_t)c, 0);  // .x: the low nibble
  const float v = ldexpf(p.x, e - 127);
  return __half_as_ushort(__float2half_rn(v));
}

__device__ __forceinline__ void build_half_lut(uint16_t* lut) {
  for (int i = threadIdx.x; i < 256 * 16; i += blockDim.x) lut[i] = half_entry(i / 16, i % 16);
}

__global__ __launch_bounds__(256) void half_lut_kernel(uint16_t* __restrict__ out) { build_half_lut(out); }

// y[t][n] = sum_k fp32(table[e][c_k]) * x[t][k]: one LDS load per weight.
__global__ __launch_bounds__(256) void gemv_hlut_kernel(const uint8_t* __restrict__ w, int N, int K,
                                                        const float* __restrict__ x, int B, float* __restrict__ y) {
  __shared__ uint16_t s_lut[256 * 16];
  build_half_lut(s_lut);
  __syncthreads();
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int row0 = (blockIdx.x * 4 + wave) * kAltR;
  if (row0 >= N) return;
  const int U = K / 32;
  for (int t = 0; t < B; ++t) {
    float acc[kAltR];
#pragma unroll
    for (int r = 0; r < kAltR; ++r) acc[r] = 0.0f;
    for (int u = lane; u < U; u += kWave) {
      const float* xu = x + (int64_t)t * K + 32 * u;
#pragma unroll
      for (int r = 0; r < kAltR; ++r) {
        const uint8_t* row = w + (int64_t)min(row0 + r, N - 1) * U * 17;
        MxRaw raw;
        mx_load(row, 17u * u, raw);
        uint32_t e, c[4];
        mx_unpack(raw, e, c);
        const uint16_t* lrow = s_lut + 16 * e;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float4 xa = *reinterpret_cast<const float4*>(xu + 8 * k);
          const float4 xb = *reinterpret_cast<const float4*>(xu + 8 * k + 4);
          const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t b = (c[k] >> (8 * j)) & 0xFFu;  // elements 8k+2j (high nibble), 8k+2j+1
            acc[r] = __builtin_fmaf(__half2float(__ushort_as_half(lrow[b >> 4])), xv[2 * j], acc[r]);
            acc[r] = __builtin_fmaf(__half2float(__ushort_as_half(lrow[b & 0xFu])), xv[2 * j + 1], acc[r]);
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kAltR; ++r) {
      // (a shuffle sum here: with the DPP tree this kernel compiled to
      // code 35-65 % slower)
      const float s = wave_sum(acc[r]);
      if (lane == 0 && row0 + r < N) y[(int64_t)t * N + row0 + r] = s;
    }
  }
}

}  // namespace

hipError_t launch_q8k_quantize(const float* x, int B, int K, int8_t* q, float* d, hipStream_t s) {
  hipLaunchKernelGGL(q8k_quantize_kernel, dim3(K / 256, B), dim3(256), 0, s, x, K, q, d);
  return hipGetLastError();
}

hipError_t launch_gemv_q8(const uint8_t* w, int N, int K, const int8_t* q, const float* d, int B, float* y,
                          hipStream_t s) {
  hipLaunchKernelGGL(gemv_q8_kernel, dim3((N + 4 * kAltR - 1) / (4 * kAltR)), dim3(256), 0, s, w, N, K, q, d, B, y);
  return hipGetLastError();
}

hipError_t launch_half_lut(uint16_t* out, hipStream_t s) {
  hipLaunchKernelGGL(half_lut_kernel, dim3(1), dim3(256), 0, s, out);
  return hipGetLastError();
}

hipError_t launch_gemv_hlut(const uint8_t* w, int N, int K, const float* x, int B, float* y, hipStream_t s) {
  hipLaunchKernelGGL(gemv_hlut_kernel, dim3((N + 4 * kAltR - 1) / (4 * kAltR)), dim3(256), 0, s, w, N, K, x, B, y);
  return hipGetLastError();
}

}  // namespace moe
