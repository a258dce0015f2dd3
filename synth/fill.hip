// GPU fill of seeded synthetic expert tensors (MXFP4 and Q2_K bytes).
//
// Input generation only: this file draws bytes from the counter-based
// SplitMix64 stream (Steele, Lea and Flood, OOPSLA 2014) with the recipes
// stated in synth/__init__.py, so that the multi-GiB expert stacks can be
// created in device memory.  It holds none of the decode path's arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;
constexpr int kTagMxfp4 = 1;
constexpr int kTagQ2k = 2;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t word(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * kGolden);
}

__device__ uint64_t tensor_key(uint64_t seed, int tag, int layer, int expert, int proj) {
  uint64_t k = mix64(seed + kGolden);
  const uint64_t ids[4] = {(uint64_t)tag, (uint64_t)(int64_t)layer, (uint64_t)(int64_t)expert,
                           (uint64_t)(int64_t)proj};
  for (int j = 0; j < 4; ++j) k = mix64((k ^ ids[j]) + kGolden);
  return k;
}

// One thread writes 16 consecutive MXFP4 blocks (272 bytes = 17 x 16 B) when
// the group is complete, otherwise single bytes for the ragged tail.
__global__ void fill_mxfp4_kernel(uint8_t* __restrict__ dst, uint64_t seed, int layer, int expert0,
                                  int proj, int64_t blocks_per_expert, int64_t groups_per_expert) {
  const int ex = blockIdx.y;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= groups_per_expert) return;
  const uint64_t key = tensor_key(seed, kTagMxfp4, layer, expert0 + ex, proj);
  uint8_t* base = dst + (int64_t)ex * blocks_per_expert * 17;
  const int64_t b0 = g * 16;
  const int64_t nb = (blocks_per_expert - b0) < 16 ? (blocks_per_expert - b0) : 16;
  if (nb == 16) {
    uint32_t out[68];
#pragma unroll
    for (int j = 0; j < 68; ++j) out[j] = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint64_t i = (uint64_t)(b0 + j);
      const uint64_t w0 = word(key, 3 * i), w1 = word(key, 3 * i + 1), w2 = word(key, 3 * i + 2);
      uint8_t bytes[17];
      bytes[0] = (uint8_t)(118u + (uint32_t)(((w2 >> 32) * 17ull) >> 32));
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        bytes[1 + t] = (uint8_t)(w0 >> (8 * t));
        bytes[9 + t] = (uint8_t)(w1 >> (8 * t));
      }
#pragma unroll
      for (int t = 0; t < 17; ++t) {
        const int pos = 17 * j + t;
        out[pos >> 2] |= (uint32_t)bytes[t] << (8 * (pos & 3));
      }
    }
    uint4* d4 = reinterpret_cast<uint4*>(base + b0 * 17);
#pragma unroll
    for (int j = 0; j < 17; ++j) d4[j] = make_uint4(out[4 * j], out[4 * j + 1], out[4 * j + 2], out[4 * j + 3]);
  } else {
    for (int64_t j = 0; j < nb; ++j) {
      const uint64_t i = (uint64_t)(b0 + j);
      const uint64_t w0 = word(key, 3 * i), w1 = word(key, 3 * i + 1), w2 = word(key, 3 * i + 2);
      uint8_t* p = base + (b0 + j) * 17;
      p[0] = (uint8_t)(118u + (uint32_t)(((w2 >> 32) * 17ull) >> 32));
      for (int t = 0; t < 8; ++t) {
        p[1 + t] = (uint8_t)(w0 >> (8 * t));
        p[9 + t] = (uint8_t)(w1 >> (8 * t));
      }
    }
  }
}

__device__ __forceinline__ uint16_t small_uniform_f16_bits(uint64_t w) {
#pragma clang fp contract(off)
  const float a = __uint_as_float(0x3A83126Fu);  // fp32 nearest 1e-3
  const float b = __uint_as_float(0x3C1374BCu);  // fp32 nearest 9e-3
  const float u = (float)(uint32_t)(w >> 40) * 5.9604644775390625e-8f;  // exact: < 2^24 times 2^-24
  const float t = b * u;
  const float v = a + t;
  const _Float16 h = (_Float16)v;
  return __builtin_bit_cast(uint16_t, h);
}

// One thread writes one Q2_K block (84 bytes = 21 dwords).
__global__ void fill_q2k_kernel(uint8_t* __restrict__ dst, uint64_t seed, int layer, int expert0,
                                int proj, int64_t blocks_per_expert) {
  const int ex = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= blocks_per_expert) return;
  const uint64_t key = tensor_key(seed, kTagQ2k, layer, expert0 + ex, proj);
  uint32_t* d = reinterpret_cast<uint32_t*>(dst + ((int64_t)ex * blocks_per_expert + i) * 84);
#pragma unroll
  for (int j = 0; j < 10; ++j) {
    const uint64_t w = word(key, 12 * (uint64_t)i + j);
    d[2 * j] = (uint32_t)w;
    d[2 * j + 1] = (uint32_t)(w >> 32);
  }
  const uint16_t hd = small_uniform_f16_bits(word(key, 12 * (uint64_t)i + 10));
  const uint16_t hm = small_uniform_f16_bits(word(key, 12 * (uint64_t)i + 11));
  d[20] = (uint32_t)hd | ((uint32_t)hm << 16);
}

}  // namespace

extern "C" int synth_fill_mxfp4(void* dst, uint64_t seed, int layer, int expert0, int n_experts,
                                int proj, int64_t blocks_per_expert, void* stream) {
  if (n_experts <= 0 || blocks_per_expert <= 0) return 0;
  // The 272-byte group stores need a 16-byte aligned base for every expert.
  if (((uintptr_t)dst & 15) != 0) return (int)hipErrorInvalidValue;
  if (((blocks_per_expert * 17) & 15) != 0 && n_experts > 1) return (int)hipErrorInvalidValue;
  const int64_t groups = (blocks_per_expert + 15) / 16;
  dim3 grid((unsigned)((groups + 255) / 256), (unsigned)n_experts);
  hipLaunchKernelGGL(fill_mxfp4_kernel, grid, dim3(256), 0, (hipStream_t)stream, (uint8_t*)dst, seed,
                     layer, expert0, proj, blocks_per_expert, groups);
  return (int)hipGetLastError();
}

extern "C" int synth_fill_q2k(void* dst, uint64_t seed, int layer, int expert0, int n_experts,
                              int proj, int64_t blocks_per_expert, void* stream) {
  if (n_experts <= 0 || blocks_per_expert <= 0) return 0;
  if (((uintptr_t)dst & 3) != 0) return (int)hipErrorInvalidValue;
  dim3 grid((unsigned)((blocks_per_expert + 255) / 256), (unsigned)n_experts);
  hipLaunchKernelGGL(fill_q2k_kernel, grid, dim3(256), 0, (hipStream_t)stream, (uint8_t*)dst, seed,
                     layer, expert0, proj, blocks_per_expert);
  return (int)hipGetLastError();
}
