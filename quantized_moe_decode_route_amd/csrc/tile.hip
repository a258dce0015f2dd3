// Block permutation from the row-major weight layout to MOE_LAYOUT_TILE256
// (one-time preparation of the down projections).  One thread per element;
// the copy is a plain gather of whole 2- or 4-byte elements.
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

}  // namespace

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
