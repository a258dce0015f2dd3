// Block permutations from the row-major weight layout to MOE_LAYOUT_TILE256
// and MOE_LAYOUT_MFMA16 (one-time preparation of the down projections).  One
// thread per destination element; each copy is a plain gather.
#include "moe_internal.h"

namespace moe {
namespace {

template <class T>
__global__ __launch_bounds__(256) void tile_rows_kernel(const T* __restrict__ src, T* __restrict__ dst, int64_t N,
                                                        int tiles, int tile) {
  const int64_t total = N * tiles * tile;
  for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < total; o += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = o % tile;
    const int64_t cn = o / tile;  // c * N + n
    const int64_t n = cn % N, c = cn / N;
    dst[o] = src[(n * tiles + c) * tile + i];
  }
}

// One thread per destination byte: block b of the MFMA16 matrix is block
// (n, j) of the row-major one, found by inverting mfma16_block.
__global__ __launch_bounds__(256) void tile_mfma16_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                          int N, int K) {
  const int JB = K / 32;  // blocks per row
  const int64_t total = (int64_t)N * JB * 17;
  for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < total; o += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = o / 17;
    const int byte = (int)(o - b * 17);
    const int i = (int)(b & 15), q = (int)((b >> 4) & 3), h = (int)((b >> 6) & 1);
    const int64_t cg = b >> 7;  // c * N/16 + n/16
    const int64_t c = cg / (N >> 4), g = cg - c * (N >> 4);
    const int64_t n = g * 16 + i;
    const int64_t j = c * 8 + h * 4 + q;
    dst[o] = src[(n * JB + j) * 17 + byte];
  }
}

}  // namespace

hipError_t launch_tile_mfma16(const uint8_t* src, uint8_t* dst, int N, int K, hipStream_t s) {
  const int64_t total = (int64_t)N * (K / 32) * 17;
  if (total <= 0) return hipSuccess;
  const int64_t blocks64 = (total + 255) / 256;
  const unsigned blocks = (unsigned)(blocks64 < 65536 ? blocks64 : 65536);
  hipLaunchKernelGGL(tile_mfma16_kernel, dim3(blocks), dim3(256), 0, s, src, dst, N, K);
  return hipGetLastError();
}

hipError_t launch_tile_rows(const void* src, void* dst, int64_t N, int tiles, int tile_elems, int elem_bytes,
                            hipStream_t s) {
  const int64_t total = N * tiles * tile_elems;
  if (total <= 0) return hipSuccess;
  const int64_t blocks64 = (total + 255) / 256;
  const unsigned blocks = (unsigned)(blocks64 < 65536 ? blocks64 : 65536);
  if (elem_bytes == 4) {
    hipLaunchKernelGGL(tile_rows_kernel<uint32_t>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), N, tiles, tile_elems);
  } else if (elem_bytes == 2) {
    hipLaunchKernelGGL(tile_rows_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), N, tiles, tile_elems);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
