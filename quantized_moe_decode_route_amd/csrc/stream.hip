// Streaming-read probe: reads a byte range once with one of the layer
// kernel's load patterns and folds every loaded dword into an XOR per
// workgroup, so its rate is a pure-read ceiling for that pattern on the
// device (the yardstick the layer's effective bandwidth is compared with).
//
//   MOE_STREAM_DWORDX4  16 bytes per lane, consecutive lanes reading
//                       consecutive 16-byte chunks
//   MOE_STREAM_MXFP4    17-byte MXFP4 blocks as the matvecs read them: lane l
//                       loads the five dwords covering block l (a dwordx4 at
//                       4-byte alignment and one dword), consecutive lanes
//                       consecutive blocks
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kUnroll = 4;  // independent loads in flight per thread

__device__ __forceinline__ uint32_t wg_xor(uint32_t v, uint32_t* s) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v ^= (uint32_t)__shfl_xor((int)v, m, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) s[threadIdx.x / kWave] = v;
  __syncthreads();
  uint32_t r = 0;
  for (int w = 0; w < kStreamThreads / kWave; ++w) r ^= s[w];
  return r;
}

__global__ __launch_bounds__(kStreamThreads) void stream_x4_kernel(const uint4* __restrict__ src, int64_t n16,
                                                                   uint32_t* __restrict__ sink) {
  __shared__ uint32_t s[kStreamThreads / kWave];
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  const uint32_t r = wg_xor(acc, s);
  if (threadIdx.x == 0) sink[blockIdx.x] = r;
}

__global__ __launch_bounds__(kStreamThreads) void stream_mx_kernel(const uint8_t* __restrict__ src, int64_t nb,
                                                                   uint32_t* __restrict__ sink) {
  __shared__ uint32_t s[kStreamThreads / kWave];
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  uint32_t acc = 0;
  int64_t b = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  auto fold = [&](const MxRaw& r) { acc ^= r.d[0] ^ r.d[1] ^ r.d[2] ^ r.d[3] ^ r.d[4]; };
  for (; b + (kUnroll - 1) * stride < nb; b += kUnroll * stride) {
    MxRaw r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t o = 17 * (b + u * stride);
      mx_load(src + (o & ~(int64_t)3), (uint32_t)(o & 3), r[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) fold(r[u]);
  }
  for (; b < nb; b += stride) {
    MxRaw r;
    const int64_t o = 17 * b;
    mx_load(src + (o & ~(int64_t)3), (uint32_t)(o & 3), r);
    fold(r);
  }
  const uint32_t r = wg_xor(acc, s);
  if (threadIdx.x == 0) sink[blockIdx.x] = r;
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, int pattern, uint32_t* sink, hipStream_t s) {
  if (pattern == MOE_STREAM_DWORDX4) {
    hipLaunchKernelGGL(stream_x4_kernel, dim3(MOE_STREAM_GRID), dim3(kStreamThreads), 0, s,
                       static_cast<const uint4*>(src), bytes / 16, sink);
  } else {
    hipLaunchKernelGGL(stream_mx_kernel, dim3(MOE_STREAM_GRID), dim3(kStreamThreads), 0, s,
                       static_cast<const uint8_t*>(src), moe_stream_mxfp4_blocks(bytes), sink);
  }
  return hipGetLastError();
}

}  // namespace moe
