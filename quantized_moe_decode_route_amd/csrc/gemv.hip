// Quantized matvec kernels: stand-alone y = W x for B tokens, and the two
// expert phases of a MoE layer (gate/up with SiLU gating, down).
//
// Mapping: one wave computes R rows.  Lane l handles the row's "units"
// l, l+64, ... (a unit is one MXFP4 block, one INT4 group, or a quarter of a
// Q2_K block, i.e. 32/32/64 weights), so each load instruction of a wave
// covers 64 consecutive units of a row: fully used cache lines.  The R rows'
// raw units are loaded first, then reused for every token; the per-lane
// partial dots are summed across the wave at the end.
#include "moe_internal.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- per-format units

struct MxFmt {
  static constexpr int kUnitW = 32;
  struct Row { const uint8_t* p; };
  struct Raw { MxRaw r; };
  static __device__ __forceinline__ Row row(const uint8_t* base, const uint16_t*, int64_t n, int K) {
    return Row{base + n * (int64_t)(K / 32) * 17};
  }
  static __device__ __forceinline__ int units(int K) { return K / 32; }
  static __device__ __forceinline__ void load(const Row& rw, int u, Raw& raw) { mx_load(rw.p, 17u * u, raw.r); }
  static __device__ __forceinline__ float dot(const Raw& raw, const float* __restrict__ x, int u) {
    uint32_t e, q[4];
    mx_unpack(raw.r, e, q);
    return e8m0_to_f32(e) * mx_block_dot(q, x + 32 * u);
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
  static __device__ __forceinline__ float dot(const Raw& raw, const float* __restrict__ x, int u) {
    const float* x64 = x + 64 * u;
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
  static __device__ __forceinline__ float dot(const Raw& raw, const float* __restrict__ x, int u) {
    const float* x32 = x + 32 * u;
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

// acc[r] = dot of row r with one token's activation x, over the whole row.
// Tokens that share rows call this once each; the repeated reads of the same
// rows by the same wave are served by the caches.
template <class F, int R>
__device__ __forceinline__ void rows_dot(const typename F::Row (&rows)[R], int K, const float* __restrict__ x,
                                         float (&acc)[R]) {
  const int U = F::units(K);
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
  for (int u = lane_id(); u < U; u += kWave) {
    typename F::Raw raw[R];
#pragma unroll
    for (int r = 0; r < R; ++r) F::load(rows[r], u, raw[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] += F::dot(raw[r], x, u);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
}

// ---------------------------------------------------------------- stand-alone matvec

constexpr int kGemvR = 2;  // rows per wave

template <class F>
__global__ __launch_bounds__(256) void gemv_kernel(const uint8_t* __restrict__ w, const uint16_t* __restrict__ sc,
                                                   int N, int K, const float* __restrict__ x, int B,
                                                   float* __restrict__ y) {
  const int wave = threadIdx.x / kWave;
  const int row0 = (blockIdx.x * 4 + wave) * kGemvR;
  if (row0 >= N) return;
  typename F::Row rows[kGemvR];
#pragma unroll
  for (int r = 0; r < kGemvR; ++r) rows[r] = F::row(w, sc, min(row0 + r, N - 1), K);
  for (int t = 0; t < B; ++t) {
    float acc[kGemvR];
    rows_dot<F, kGemvR>(rows, K, x + (int64_t)t * K, acc);
    if (lane_id() == 0) {
#pragma unroll
      for (int r = 0; r < kGemvR; ++r)
        if (row0 + r < N) y[(int64_t)t * N + row0 + r] = acc[r];
    }
  }
}

// ---------------------------------------------------------------- layer phases

constexpr int kGateUpR = 4;  // gate rows (and as many up rows) per wave
constexpr int kDownR = 4;

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// grid = (ceil(F / (4 * kGateUpR)), B * k); block y is a unique-expert slot.
template <class F>
__global__ __launch_bounds__(256) void gate_up_kernel(WeightRef gate, WeightRef up, int D, int Fd, int k,
                                                      uint8_t* __restrict__ ws, WsLayout L) {
  const int g = blockIdx.y;
  const int U = *reinterpret_cast<const int32_t*>(ws + L.ngroups);
  if (g >= U) return;
  const ExpertGroup grp = reinterpret_cast<const ExpertGroup*>(ws + L.groups)[g];
  const int wave = threadIdx.x / kWave;
  const int row0 = (blockIdx.x * 4 + wave) * kGateUpR;
  if (row0 >= Fd) return;
  const uint8_t* gbase = gate.base + grp.expert * gate.stride;
  const uint8_t* ubase = up.base + grp.expert * up.stride;
  const uint16_t* gs = gate.scale ? reinterpret_cast<const uint16_t*>(
                                        reinterpret_cast<const uint8_t*>(gate.scale) + grp.expert * gate.scale_stride)
                                  : nullptr;
  const uint16_t* us = up.scale ? reinterpret_cast<const uint16_t*>(
                                      reinterpret_cast<const uint8_t*>(up.scale) + grp.expert * up.scale_stride)
                                : nullptr;
  typename F::Row rows[2 * kGateUpR];
#pragma unroll
  for (int r = 0; r < kGateUpR; ++r) {
    rows[r] = F::row(gbase, gs, min(row0 + r, Fd - 1), D);
    rows[kGateUpR + r] = F::row(ubase, us, min(row0 + r, Fd - 1), D);
  }
  const float* xf = reinterpret_cast<const float*>(ws + L.xf);
  float* h = reinterpret_cast<float*>(ws + L.h);
  for (int t = 0; t < grp.n; ++t) {
    float acc[2 * kGateUpR];
    rows_dot<F, 2 * kGateUpR>(rows, D, xf + (int64_t)grp.tok[t] * D, acc);
    if (lane_id() == 0) {
      float* hrow = h + ((int64_t)grp.tok[t] * k + grp.slot[t]) * Fd;
#pragma unroll
      for (int r = 0; r < kGateUpR; ++r)
        if (row0 + r < Fd) hrow[row0 + r] = silu(acc[r]) * acc[kGateUpR + r];
    }
  }
}

// grid = (ceil(D / (4 * kDownR)), B * k).
template <class F>
__global__ __launch_bounds__(256) void down_kernel(WeightRef down, int D, int Fd, int k, uint8_t* __restrict__ ws,
                                                   WsLayout L) {
  const int g = blockIdx.y;
  const int U = *reinterpret_cast<const int32_t*>(ws + L.ngroups);
  if (g >= U) return;
  const ExpertGroup grp = reinterpret_cast<const ExpertGroup*>(ws + L.groups)[g];
  const int wave = threadIdx.x / kWave;
  const int row0 = (blockIdx.x * 4 + wave) * kDownR;
  if (row0 >= D) return;
  const uint8_t* dbase = down.base + grp.expert * down.stride;
  const uint16_t* ds = down.scale ? reinterpret_cast<const uint16_t*>(
                                        reinterpret_cast<const uint8_t*>(down.scale) + grp.expert * down.scale_stride)
                                  : nullptr;
  typename F::Row rows[kDownR];
#pragma unroll
  for (int r = 0; r < kDownR; ++r) rows[r] = F::row(dbase, ds, min(row0 + r, D - 1), Fd);
  const float* h = reinterpret_cast<const float*>(ws + L.h);
  float* yp = reinterpret_cast<float*>(ws + L.yp);
  for (int t = 0; t < grp.n; ++t) {
    const int64_t ts = (int64_t)grp.tok[t] * k + grp.slot[t];
    float acc[kDownR];
    rows_dot<F, kDownR>(rows, Fd, h + ts * Fd, acc);
    if (lane_id() == 0) {
#pragma unroll
      for (int r = 0; r < kDownR; ++r)
        if (row0 + r < D) yp[ts * D + row0 + r] = acc[r];
    }
  }
}

}  // namespace

#define MOE_DISPATCH(KERNEL, grid, s, ...)                                                  \
  switch (fmt) {                                                                            \
    case MOE_FMT_MXFP4: hipLaunchKernelGGL(KERNEL<MxFmt>, grid, dim3(256), 0, s, __VA_ARGS__); break;    \
    case MOE_FMT_Q2K: hipLaunchKernelGGL(KERNEL<Q2kFmt>, grid, dim3(256), 0, s, __VA_ARGS__); break;    \
    case MOE_FMT_INT4G32: hipLaunchKernelGGL(KERNEL<Int4Fmt>, grid, dim3(256), 0, s, __VA_ARGS__); break; \
    default: return hipErrorInvalidValue;                                                   \
  }                                                                                         \
  return hipGetLastError();

hipError_t launch_gemv(int fmt, const void* w0, const uint16_t* scale, int N, int K, const float* x, int B,
                       float* y, hipStream_t s) {
  const int rows_per_block = 4 * kGemvR;
  dim3 grid((N + rows_per_block - 1) / rows_per_block);
  const uint8_t* w = static_cast<const uint8_t*>(w0);
  MOE_DISPATCH(gemv_kernel, grid, s, w, scale, N, K, x, B, y)
}

hipError_t launch_gate_up(int fmt, const WeightRef& gate, const WeightRef& up, int D, int F, int B, int k,
                          uint8_t* ws, const WsLayout& L, hipStream_t s) {
  dim3 grid((F + 4 * kGateUpR - 1) / (4 * kGateUpR), B * k);
  MOE_DISPATCH(gate_up_kernel, grid, s, gate, up, D, F, k, ws, L)
}

hipError_t launch_down(int fmt, const WeightRef& down, int D, int F, int B, int k, uint8_t* ws, const WsLayout& L,
                       hipStream_t s) {
  dim3 grid((D + 4 * kDownR - 1) / (4 * kDownR), B * k);
  MOE_DISPATCH(down_kernel, grid, s, down, D, F, k, ws, L)
}

}  // namespace moe
