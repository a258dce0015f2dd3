// FP4 (MXFP4) -> INT4 group-32 conversion with the six-candidate scale
// search of the DeepSeek-V4-Flash-0731-W4A16 model card ("FP4 -> INT4
// conversion algorithm", steps 1 and 2), and the MXFP4 exponent validator.
//
// Decisions (rounding of w/s, the argmin over candidates) are taken in the
// precisions the method fixes: fp32 for the scale, the quotient, rint and
// the clamp; the squared error is summed in fp64 in index order.  Contraction
// of multiply-add pairs is off so every operation rounds once, as written.
#include "moe_internal.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

// fp32 values of the Python doubles 6/7, 0.9, 0.95, 1.0, 1.05, 1.1.
__constant__ uint32_t kCandBits[6] = {0x3F5B6DB7u, 0x3F666666u, 0x3F733333u,
                                      0x3F800000u, 0x3F866666u, 0x3F8CCCCDu};

// One thread per 32-weight group (= one MXFP4 block).
__global__ __launch_bounds__(256) void quantize_kernel(const uint8_t* __restrict__ mx, int64_t ngroups,
                                                       int32_t* __restrict__ qout, uint16_t* __restrict__ sout) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= ngroups) return;
  // mx is 4-byte aligned; block g starts at byte 17g of it (4 blocks = 68 B
  // keep 4-byte alignment, so address from the group of four).
  MxRaw raw;
  mx_load(mx + (g & ~(int64_t)3) * 17, (uint32_t)(17 * (g & 3)), raw);
  uint32_t e, q[4];
  mx_unpack(raw, e, q);
  const float scale = e8m0_to_f32(e);
  float w[32];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f32x2 p[4] = {MOE_FP4X2(q[d], 0), MOE_FP4X2(q[d], 1), MOE_FP4X2(q[d], 2), MOE_FP4X2(q[d], 3)};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int j = 4 * d + b;       // code byte j
      w[2 * j] = p[b].y * scale;     // high nibble: element 2j
      w[2 * j + 1] = p[b].x * scale; // low nibble: element 2j+1
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(w[i]));
  const float floor_amax = __uint_as_float(0x322BCC77u);  // fp32 nearest 1e-8
  if (amax < floor_amax) amax = floor_amax;

  double best_err = __builtin_inf();
  float best_s = 0.0f;
  uint32_t best_words[4] = {0u, 0u, 0u, 0u};
  for (int c = 0; c < 6; ++c) {
    const float prod = amax * __uint_as_float(kCandBits[c]);
    const float s = prod / 7.0f;
    double err = 0.0;
    uint32_t words[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float r = __builtin_rintf(w[i] / s);
      r = fminf(fmaxf(r, -8.0f), 7.0f);
      const int qi = (int)r;
      words[i / 8] |= ((uint32_t)qi & 0xFu) << (4 * (i % 8));
      const double diff = (double)w[i] - (double)qi * (double)s;
      err = err + diff * diff;
    }
    if (err < best_err) {
      best_err = err;
      best_s = s;
#pragma unroll
      for (int i = 0; i < 4; ++i) best_words[i] = words[i];
    }
  }
  *reinterpret_cast<uint4*>(qout + 4 * g) = make_uint4(best_words[0], best_words[1], best_words[2], best_words[3]);
  sout[g] = (uint16_t)f32_to_bf16_rne(best_s);
}

__global__ __launch_bounds__(256) void validate_kernel(const uint8_t* __restrict__ blocks, int64_t n,
                                                       int32_t* __restrict__ bad) {
  int cnt = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    cnt += blocks[17 * i] == 0xFF;
  cnt = (int)wave_sum((float)cnt);
  if (lane_id() == 0 && cnt) atomicAdd(bad, cnt);
}

}  // namespace

hipError_t launch_quantize_int4(const uint8_t* mx, int64_t ngroups, int32_t* q, uint16_t* scale, hipStream_t s) {
  if (ngroups == 0) return hipSuccess;
  dim3 grid((unsigned)((ngroups + 255) / 256));
  hipLaunchKernelGGL(quantize_kernel, grid, dim3(256), 0, s, mx, ngroups, q, scale);
  return hipGetLastError();
}

hipError_t launch_validate_mxfp4(const uint8_t* blocks, int64_t n, int32_t* bad, hipStream_t s) {
  if (n == 0) return hipSuccess;
  int64_t want = (n + 255) / 256;
  dim3 grid((unsigned)(want < 4096 ? want : 4096));
  hipLaunchKernelGGL(validate_kernel, grid, dim3(256), 0, s, blocks, n, bad);
  return hipGetLastError();
}

}  // namespace moe
