// Quantized matvec kernels: stand-alone y = W x for B tokens, and the two
// expert phases of a MoE layer (gate/up with SiLU gating, down).
//
// Mapping: one wave computes R rows.  Lane l handles the row's "units"
// l, l+64, ... (a unit is one MXFP4 block, one INT4 group, or a quarter of a
// Q2_K block, i.e. 32/32/64 weights), so each load instruction of a wave
// covers 64 consecutive units of a row: fully used cache lines.  The R rows'
// raw units are loaded first, then reused for every token; the per-lane
// partial dots are summed across the wave at the end.
#include <type_traits>

#include "units.h"

namespace moe {
namespace {

// acc[r] = dot of row r with one token's activation x, over the whole row.
// Tokens that share rows call this once each; the repeated reads of the same
// rows by the same wave are served by the caches (the stand-alone matvec
// keeps short rows in registers instead, gemv_regs_kernel, and passes over
// long rows once per four tokens, rows_dot_tokens).
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
    for (int r = 0; r < R; ++r) acc[r] += F::dot(raw[r], (uint32_t)u & 3u, x + (int64_t)F::kUnitW * u);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
}

// rows_dot for TT tokens at once (token j's activation at x + j * K): each
// unit of the rows is loaded once for the TT tokens, and every token's sum
// is taken in rows_dot's order, so its bits are rows_dot's.
template <class F, int R, int TT>
__device__ __forceinline__ void rows_dot_tokens(const typename F::Row (&rows)[R], int K,
                                                const float* __restrict__ x, float (&acc)[TT][R]) {
  const int U = F::units(K);
#pragma unroll
  for (int j = 0; j < TT; ++j)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[j][r] = 0.0f;
  for (int u = lane_id(); u < U; u += kWave) {
    typename F::Raw raw[R];
#pragma unroll
    for (int r = 0; r < R; ++r) F::load(rows[r], u, raw[r]);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < TT; ++j)
        acc[j][r] += F::dot(raw[r], (uint32_t)u & 3u, x + (int64_t)j * K + (int64_t)F::kUnitW * u);
  }
#pragma unroll
  for (int j = 0; j < TT; ++j)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[j][r] = wave_sum(acc[j][r]);
}

// Same for rows n[r] of a matrix [N][K] stored in MOE_LAYOUT_TILE256: unit u
// of row n is unit u % UPT of row (u / UPT) * N + n of the [(K/256)*N][256]
// matrix.
template <class F, int R>
__device__ __forceinline__ void rows_dot_tiled(const uint8_t* base, const uint16_t* sc, const int (&n)[R], int N,
                                               int K, const float* __restrict__ x, float (&acc)[R]) {
  constexpr int UPT = kTileCols / F::kUnitW;
  const int U = F::units(K);
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
  for (int u = lane_id(); u < U; u += kWave) {
    const int c = u / UPT, uu = u % UPT;
    typename F::Raw raw[R];
#pragma unroll
    for (int r = 0; r < R; ++r) F::load(F::row(base, sc, (int64_t)c * N + n[r], kTileCols), uu, raw[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] += F::dot(raw[r], (uint32_t)uu & 3u, x + (int64_t)F::kUnitW * u);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
}

// Same for MXFP4 rows stored in MOE_LAYOUT_MFMA16 (block j of row n is
// block mfma16_block(n, j, N) of the matrix).
template <int R>
__device__ __forceinline__ void rows_dot_mfma16(const uint8_t* base, const int (&n)[R], int N, int K,
                                                const float* __restrict__ x, float (&acc)[R]) {
  const int U = K / 32;
  const MxFmt::Row all{base};
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
  for (int u = lane_id(); u < U; u += kWave) {
    MxFmt::Raw raw[R];
    int b[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      b[r] = (int)mfma16_block(n[r], u, N);
      MxFmt::load(all, b[r], raw[r]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] += MxFmt::dot(raw[r], (uint32_t)b[r] & 3u, x + (int64_t)32 * u);
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
  int t = 0;
  for (; t + 4 <= B; t += 4) {  // four tokens per pass over the rows
    float acc[4][kGemvR];
    rows_dot_tokens<F, kGemvR, 4>(rows, K, x + (int64_t)t * K, acc);
    if (lane_id() == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < kGemvR; ++r)
          if (row0 + r < N) y[(int64_t)(t + j) * N + row0 + r] = acc[j][r];
    }
  }
  for (; t < B; ++t) {
    float acc[kGemvR];
    rows_dot<F, kGemvR>(rows, K, x + (int64_t)t * K, acc);
    if (lane_id() == 0) {
#pragma unroll
      for (int r = 0; r < kGemvR; ++r)
        if (row0 + r < N) y[(int64_t)t * N + row0 + r] = acc[r];
    }
  }
}

constexpr int kGemvXs = 16384;  // fp32 activations staged per chunk of tokens
constexpr int kGemvThreads = 256;  // the stand-alone matvec's workgroup size

// The dots of a wave's kGemvR register-held rows with TT consecutive staged
// tokens (slots s0.. of the chunk, tokens t.. of the call), stored to y.  The
// TT tokens' accumulations are independent chains, so they overlap; each
// token still adds its units in ascending order and then sums over the wave
// (one fixed DPP tree), so its result has the same bits whatever TT is.  A unit's decode does not
// depend on the activations and is shared by the TT tokens.
template <class F, int UPL, int TT>
__device__ __forceinline__ void regs_tokens(const typename F::Raw (&raw)[kGemvR][UPL], const float* xs, int K, int s0,
                                            int t, int N, int row0, float* __restrict__ y) {
  constexpr int C = F::kUnitW / 4;
  const int U = F::units(K), lane = lane_id();
  float acc[TT][kGemvR];
#pragma unroll
  for (int j = 0; j < TT; ++j)
#pragma unroll
    for (int r = 0; r < kGemvR; ++r) acc[j][r] = 0.0f;
#pragma unroll
  for (int i = 0; i < UPL; ++i) {
    const int u = lane + kWave * i;
    if (u < U) {
      float xv[TT][F::kUnitW];
#pragma unroll
      for (int j = 0; j < TT; ++j) {
        const float4* xt4 = reinterpret_cast<const float4*>(xs) + (s0 + j) * (K / 4) + u;
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const float4 v = xt4[c * U];
          xv[j][4 * c] = v.x;
          xv[j][4 * c + 1] = v.y;
          xv[j][4 * c + 2] = v.z;
          xv[j][4 * c + 3] = v.w;
        }
      }
#pragma unroll
      for (int r = 0; r < kGemvR; ++r)
#pragma unroll
        for (int j = 0; j < TT; ++j) acc[j][r] += F::dot(raw[r][i], (uint32_t)u & 3u, xv[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < TT; ++j)
#pragma unroll
    for (int r = 0; r < kGemvR; ++r) acc[j][r] = wave_sum_dpp(acc[j][r]);
  if (lane == kWave - 1) {  // where the DPP tree leaves the sums
#pragma unroll
    for (int j = 0; j < TT; ++j)
#pragma unroll
      for (int r = 0; r < kGemvR; ++r)
        if (row0 + r < N) y[(int64_t)(t + j) * N + row0 + r] = acc[j][r];
  }
}

// The same matvec with the wave's weights held in registers: every lane
// first requests all of its units of the kGemvR rows (UPL units per row, one
// memory round trip), then each token's dots run from those registers, so
// the weights are loaded once whatever B is.  The workgroup stages the
// activations of as many tokens as fit in LDS (64 KB) at a time, so a
// token's dots wait for LDS rather than for one L2 round trip per token.
// Per token a lane adds its units in ascending order, then the wave sums in
// a fixed DPP tree, so a token's result does not depend on B; staged
// tokens are taken up to four at a time (regs_tokens), which keeps up to
// eight independent accumulations in flight on the one wave of each SIMD.
template <class F, int UPL>
__global__ __launch_bounds__(kGemvThreads) void gemv_regs_kernel(const uint8_t* __restrict__ w, const uint16_t* __restrict__ sc,
                                                        int N, int K, const float* __restrict__ x, int B,
                                                        float* __restrict__ y) {
  __shared__ __align__(16) float xs[kGemvXs];
  const int wave = threadIdx.x / kWave;
  const int row0 = (blockIdx.x * 4 + wave) * kGemvR;
  const bool rows_here = row0 < N;  // waves without rows still stage activations
  const int U = F::units(K);
  const int lane = lane_id();
  // tokens per group: as many as the registers hold without spilling (the
  // staged activations of a group take TT * kUnitW registers)
  constexpr int kTok = F::kUnitW >= 64 ? (UPL >= 2 ? 1 : 2) : 4;
  typename F::Raw raw[kGemvR][UPL];
#pragma unroll
  for (int r = 0; r < kGemvR; ++r) {
    const typename F::Row row = F::row(w, sc, min(min(row0, N - 1) + r, N - 1), K);
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
      const int u = lane + kWave * i;
      F::load(row, u < U ? u : 0, raw[r][i]);
    }
  }
  const int tc = K <= kGemvXs ? kGemvXs / K : 0;  // tokens per chunk (0: read x from memory)
  for (int t0 = 0; t0 < B; t0 += tc > 0 ? tc : B) {
    const int nt = tc > 0 ? min(tc, B - t0) : B;
    if (tc > 0) {
      __syncthreads();  // the previous chunk is consumed
      const float4* src = reinterpret_cast<const float4*>(x + (int64_t)t0 * K);
      // chunk c (4 activations) of unit u of token t goes to float4 slot
      // t * K/4 + c * U + u: the lanes' reads of one chunk are consecutive
      constexpr int C = F::kUnitW / 4;
      const int K4 = K / 4;
      for (int i = threadIdx.x; i < nt * K4; i += blockDim.x) {
        const int t = i / K4, j = i - t * K4;
        reinterpret_cast<float4*>(xs)[t * K4 + (j % C) * U + j / C] = src[i];
      }
      __syncthreads();
    }
    if (!rows_here) continue;
    int t = t0;
    if (tc > 0) {  // staged tokens: kTok (then fewer) at a time
      if constexpr (kTok >= 4)
        for (; t + 4 <= t0 + nt; t += 4) regs_tokens<F, UPL, 4>(raw, xs, K, t - t0, t, N, row0, y);
      if constexpr (kTok >= 2)
        for (; t + 2 <= t0 + nt; t += 2) regs_tokens<F, UPL, 2>(raw, xs, K, t - t0, t, N, row0, y);
      for (; t < t0 + nt; ++t) regs_tokens<F, UPL, 1>(raw, xs, K, t - t0, t, N, row0, y);
      continue;
    }
    for (; t < t0 + nt; ++t) {
      float acc[kGemvR];
#pragma unroll
      for (int r = 0; r < kGemvR; ++r) acc[r] = 0.0f;
#pragma unroll
      for (int i = 0; i < UPL; ++i) {
        const int u = lane + kWave * i;
        if (u < U) {
          const float* xt = x + (int64_t)t * K + (int64_t)F::kUnitW * u;
#pragma unroll
          for (int r = 0; r < kGemvR; ++r) acc[r] += F::dot(raw[r][i], (uint32_t)u & 3u, xt);
        }
      }
#pragma unroll
      for (int r = 0; r < kGemvR; ++r) acc[r] = wave_sum_dpp(acc[r]);
      if (lane == kWave - 1) {
#pragma unroll
        for (int r = 0; r < kGemvR; ++r)
          if (row0 + r < N) y[(int64_t)t * N + row0 + r] = acc[r];
      }
    }
  }
}

template <class F>
hipError_t launch_gemv_f(const uint8_t* w, const uint16_t* scale, int N, int K, const float* x, int B, float* y,
                         hipStream_t s) {
  const int rows_per_block = 4 * kGemvR;
  const dim3 grid((N + rows_per_block - 1) / rows_per_block);
  const int upl = (K / F::kUnitW + kWave - 1) / kWave;  // units per lane and row
  if (upl <= 1)
    hipLaunchKernelGGL((gemv_regs_kernel<F, 1>), grid, dim3(kGemvThreads), 0, s, w, scale, N, K, x, B, y);
  else if (upl <= 2)
    hipLaunchKernelGGL((gemv_regs_kernel<F, 2>), grid, dim3(kGemvThreads), 0, s, w, scale, N, K, x, B, y);
  else if (upl <= 4)
    hipLaunchKernelGGL((gemv_regs_kernel<F, 4>), grid, dim3(kGemvThreads), 0, s, w, scale, N, K, x, B, y);
  else  // long rows: stream them per token
    hipLaunchKernelGGL(gemv_kernel<F>, grid, dim3(256), 0, s, w, scale, N, K, x, B, y);
  return hipGetLastError();
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
  int rn[kDownR];
#pragma unroll
  for (int r = 0; r < kDownR; ++r) {
    rn[r] = min(row0 + r, D - 1);
    rows[r] = F::row(dbase, ds, rn[r], Fd);
  }
  const float* h = reinterpret_cast<const float*>(ws + L.h);
  float* yp = reinterpret_cast<float*>(ws + L.yp);
  for (int t = 0; t < grp.n; ++t) {
    const int64_t ts = (int64_t)grp.tok[t] * k + grp.slot[t];
    float acc[kDownR];
    bool done = false;
    if constexpr (std::is_same<F, MxFmt>::value) {
      if (down.layout == MOE_LAYOUT_MFMA16) {
        rows_dot_mfma16<kDownR>(dbase, rn, D, Fd, h + ts * Fd, acc);
        done = true;
      }
    }
    if (!done) {
      if (down.layout == MOE_LAYOUT_TILE256)
        rows_dot_tiled<F, kDownR>(dbase, ds, rn, D, Fd, h + ts * Fd, acc);
      else
        rows_dot<F, kDownR>(rows, Fd, h + ts * Fd, acc);
    }
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
  const uint8_t* w = static_cast<const uint8_t*>(w0);
  switch (fmt) {
    case MOE_FMT_MXFP4: return launch_gemv_f<MxFmt>(w, scale, N, K, x, B, y, s);
    case MOE_FMT_Q2K: return launch_gemv_f<Q2kFmt>(w, scale, N, K, x, B, y, s);
    case MOE_FMT_INT4G32: return launch_gemv_f<Int4Fmt>(w, scale, N, K, x, B, y, s);
    default: return hipErrorInvalidValue;
  }
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
