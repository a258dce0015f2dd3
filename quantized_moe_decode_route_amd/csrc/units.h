// Per-format "units" of a weight row for the matvec kernels: a unit is one
// MXFP4 block (32 weights), one INT4 group (32 weights) or a quarter of a
// Q2_K block (64 weights = 4 sub-blocks of 16).  Each format gives the row
// address, the raw bytes of one unit (loaded with dword-aligned vector loads)
// and the dot product of a unit with the fp32 activations of its weights.
#pragma once

#include "moe_internal.h"

namespace moe {

struct MxFmt {
  static constexpr int kUnitW = 32;
  struct Row { const uint8_t* p; };
  struct Raw { MxRaw r; };
  static __device__ __forceinline__ Row row(const uint8_t* base, const uint16_t*, int64_t n, int K) {
    return Row{base + n * (int64_t)(K / 32) * 17};
  }
  static __device__ __forceinline__ int units(int K) { return K / 32; }
  static __device__ __forceinline__ void load(const Row& rw, int u, Raw& raw) { mx_load(rw.p, 17u * u, raw.r); }
  static __device__ __forceinline__ float dot(const Raw& raw, const float* __restrict__ x32) {
    uint32_t e, q[4];
    mx_unpack(raw.r, e, q);
    return e8m0_to_f32(e) * mx_block_dot(q, x32);
  }
};

struct Q2kFmt {
  static constexpr int kUnitW = 64;  // a quarter of a 256-weight block: 4 sub-blocks of 16
  struct Row { const uint8_t* p; };
  struct Raw { uint32_t qs[4]; uint32_t sc; uint32_t dd; };
  static __device__ __forceinline__ Row row(const uint8_t* base, const uint16_t*, int64_t n, int K) {
    return Row{base + n * (int64_t)(K / 256) * 84};
  }
  static __device__ __forceinline__ int units(int K) { return K / 64; }
  static __device__ __forceinline__ void load(const Row& rw, int u, Raw& raw) {
    const uint8_t* blk = rw.p + 84 * (u >> 2);
    const int qq = u & 3;
    const uint4 v = *reinterpret_cast<const uint4*>(__builtin_assume_aligned(blk + 16 + 16 * qq, 4));
    raw.qs[0] = v.x;
    raw.qs[1] = v.y;
    raw.qs[2] = v.z;
    raw.qs[3] = v.w;
    raw.sc = *reinterpret_cast<const uint32_t*>(__builtin_assume_aligned(blk + 4 * qq, 4));
    raw.dd = *reinterpret_cast<const uint32_t*>(__builtin_assume_aligned(blk + 80, 4));
  }
  static __device__ __forceinline__ float dot(const Raw& raw, const float* __restrict__ x64) {
    const float d = f16_to_f32(raw.dd & 0xFFFFu);
    const float dmin = f16_to_f32(raw.dd >> 16);
    float acc = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float sqx = 0.0f, sx = 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 xv = *reinterpret_cast<const float4*>(x64 + 16 * s + 4 * c);
        const uint32_t b = raw.qs[s] >> (8 * c);  // byte c of sub-block s: weights 4c..4c+3
        sqx = __builtin_fmaf((float)(b & 3u), xv.x, sqx);
        sqx = __builtin_fmaf((float)((b >> 2) & 3u), xv.y, sqx);
        sqx = __builtin_fmaf((float)((b >> 4) & 3u), xv.z, sqx);
        sqx = __builtin_fmaf((float)((b >> 6) & 3u), xv.w, sqx);
        sx += (xv.x + xv.y) + (xv.z + xv.w);
      }
      const uint32_t sb = (raw.sc >> (8 * s)) & 0xFFu;
      const float scale = d * (float)(sb & 0xFu);
      const float mn = dmin * (float)(sb >> 4);
      acc = __builtin_fmaf(scale, sqx, acc);
      acc = __builtin_fmaf(-mn, sx, acc);
    }
    return acc;
  }
};

struct Int4Fmt {
  static constexpr int kUnitW = 32;
  struct Row { const uint32_t* q; const uint16_t* s; };
  struct Raw { uint32_t q[4]; uint32_t s; };
  static __device__ __forceinline__ Row row(const uint8_t* base, const uint16_t* sc, int64_t n, int K) {
    return Row{reinterpret_cast<const uint32_t*>(base) + n * (int64_t)(K / 8), sc + n * (int64_t)(K / 32)};
  }
  static __device__ __forceinline__ int units(int K) { return K / 32; }
  static __device__ __forceinline__ void load(const Row& rw, int u, Raw& raw) {
    const uint4 v = *reinterpret_cast<const uint4*>(rw.q + 4 * u);
    raw.q[0] = v.x;
    raw.q[1] = v.y;
    raw.q[2] = v.z;
    raw.q[3] = v.w;
    raw.s = rw.s[u];
  }
  static __device__ __forceinline__ float dot(const Raw& raw, const float* __restrict__ x32) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4 xa = *reinterpret_cast<const float4*>(x32 + 8 * w);
      const float4 xb = *reinterpret_cast<const float4*>(x32 + 8 * w + 4);
      const int32_t c = (int32_t)raw.q[w];
      acc = __builtin_fmaf((float)((c << 28) >> 28), xa.x, acc);
      acc = __builtin_fmaf((float)((c << 24) >> 28), xa.y, acc);
      acc = __builtin_fmaf((float)((c << 20) >> 28), xa.z, acc);
      acc = __builtin_fmaf((float)((c << 16) >> 28), xa.w, acc);
      acc = __builtin_fmaf((float)((c << 12) >> 28), xb.x, acc);
      acc = __builtin_fmaf((float)((c << 8) >> 28), xb.y, acc);
      acc = __builtin_fmaf((float)((c << 4) >> 28), xb.z, acc);
      acc = __builtin_fmaf((float)(c >> 28), xb.w, acc);
    }
    return bf16_to_f32(raw.s) * acc;
  }
};

}  // namespace moe
