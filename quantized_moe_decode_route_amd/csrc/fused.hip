// One MoE layer in a single launch: one 512-thread workgroup per compute
// unit, no grid barriers and no memory fences on the hot path.
//
// Workgroups exchange results through tagged 64-bit words: a 32-bit payload
// plus the call's epoch number.  A consumer spins on the words it needs until
// every tag equals the current epoch, so each dependency waits exactly for
// the data it consumes.  All exchanges use agent-coherent 64-bit accesses
// (workgroup-scope stores are not reliably seen by other compute units of the
// same XCD while the kernel runs).  A workgroup learns its XCD from the
// XCC_ID hardware register and its index inside the XCD from an L2-local
// counter: with one workgroup per compute unit (the LDS footprint allows no
// more), every XCD holds exactly grid/NX of them, whatever order the
// dispatcher used.
//
//  1. Routing.  Workgroup g computes expert g's router logits for every token
//     (fp64) and publishes them device-wide.  Every workgroup gathers all
//     logits and derives, identically, each token's top-k (largest first, ties
//     to the lower index), the softmax weights and the grouping of
//     (token, rank) pairs by expert.
//  2. Gate/up.  XCD x owns the d_ff slice [x*F/NX, (x+1)*F/NX): its workgroups
//     compute h = SiLU(gate.x) * (up.x) for those rows of every selected
//     expert, keeping the next two experts' blocks in flight, and publish h.
//  3. Down.  XCD x multiplies every down row's slice-x columns by its own h
//     slice (partial sums over d_ff), combines the k ranks of each token in
//     rank order, and publishes the partial outputs device-wide; the output
//     rows are then finished by summing the NX partials in XCD order.
//
// A token's arithmetic does not depend on the other tokens in the call (same
// lane mapping, same reduction trees), so B=8 rows equal B=1 results bit for
// bit.  Every wait is bounded (about 0.5 s); on timeout a flag is raised in
// the workspace and the kernel runs to completion.
#include "units.h"

namespace moe {
namespace {

constexpr int kW = 8;     // waves per workgroup
constexpr int kMaxNX = 16; // XCDs supported
constexpr int kTracePoints = 10;
constexpr uint64_t kSpinTicks = 50000000ull;  // 0.5 s of the 100 MHz wall clock

// ---------------------------------------------------------------- tagged exchange

__device__ __forceinline__ uint64_t tagged(uint32_t payload, uint32_t tag) {
  return ((uint64_t)tag << 32) | payload;
}
__device__ __forceinline__ uint32_t tag_of(uint64_t w) { return (uint32_t)(w >> 32); }
__device__ __forceinline__ uint32_t payload_of(uint64_t w) { return (uint32_t)w; }

// device-wide (agent-coherent)
__device__ __forceinline__ void st_dev(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// ---------------------------------------------------------------- DPP reductions

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF,
                                                               false));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int v, int old) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, false);
}

// Sum over the wave in a fixed tree; the total lands in lane 63.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f<0xB1>(v);        // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);        // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);       // row_half_mirror
  v += dpp_f<0x140>(v);       // row_mirror
  v += dpp_f<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_f<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

// Sum over aligned groups of G lanes (G = 1, 2, 4, 8 or 16); every lane of a
// group ends with the group's sum.
template <int G>
__device__ __forceinline__ float group_sum_dpp(float v) {
  if (G >= 2) v += dpp_f<0xB1>(v);
  if (G >= 4) v += dpp_f<0x4E>(v);
  if (G >= 8) v += dpp_f<0x141>(v);
  if (G >= 16) v += dpp_f<0x140>(v);
  return v;
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_d(double v) {
  const int lo = dpp_i<CTRL, ROW_MASK>(__double2loint(v), 0);
  const int hi = dpp_i<CTRL, ROW_MASK>(__double2hiint(v), 0);
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double wave_sum_dpp_f64(double v) {
  v += dpp_d<0xB1>(v);
  v += dpp_d<0x4E>(v);
  v += dpp_d<0x141>(v);
  v += dpp_d<0x140>(v);
  v += dpp_d<0x142, 0xA>(v);
  v += dpp_d<0x143, 0xC>(v);
  return v;
}

// (value, index) with "better" = larger value, then lower index.
__device__ __forceinline__ bool better(double va, int ia, double vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ void argmax_step(double& v, int& i) {
  // Lanes without a source read (-inf, INT_MAX), which never wins.
  const int lo = dpp_i<CTRL, ROW_MASK>(__double2loint(v), 0);
  const int hi = dpp_i<CTRL, ROW_MASK>(__double2hiint(v), (int)0xFFF00000);
  const int oi = dpp_i<CTRL, ROW_MASK>(i, 0x7FFFFFFF);
  const double ov = __hiloint2double(hi, lo);
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

// Wave-wide best (value, index), returned uniformly to all lanes.
__device__ __forceinline__ void wave_argmax(double& v, int& i) {
  argmax_step<0xB1>(v, i);
  argmax_step<0x4E>(v, i);
  argmax_step<0x141>(v, i);
  argmax_step<0x140>(v, i);
  argmax_step<0x142, 0xA>(v, i);
  argmax_step<0x143, 0xC>(v, i);
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), 63);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), 63);
  i = __builtin_amdgcn_readlane(i, 63);
  v = __hiloint2double(hi, lo);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

struct FusedArgs {
  const float* router_w;
  const uint16_t* x;  // bf16 bits [B][D]
  WeightRef gate, up, down;
  uint8_t* ws;
  WsLayout L;
  float* y;
  const float* residual;
  int32_t* idx_out;
  float* gw_out;
  uint64_t* trace;
  int E, D, Fd, k, B;
  int nx;  // XCDs (the grid holds grid/nx workgroups on each)
};

__device__ __forceinline__ uint32_t xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xFu;  // HW_REG_XCC_ID bits 3:0
}

__device__ __forceinline__ void stamp(const FusedArgs& a, int point) {
  if (a.trace && threadIdx.x == 0) a.trace[blockIdx.x * kTracePoints + point] = wall_clock64();
}

// LDS shared by the phases (activations during gate/up; h slices and row
// partials during down).
constexpr int kLdsBytes = 128 * 1024;

template <class F, int MAXU>
__device__ __forceinline__ void load_pair(const typename F::Row& r0, const typename F::Row& r1, int U, int lane,
                                          typename F::Raw (&raw)[MAXU][2]) {
#pragma unroll
  for (int j = 0; j < MAXU; ++j) {
    const int u = lane + kWave * j;
    if (u < U) {
      F::load(r0, u, raw[j][0]);
      F::load(r1, u, raw[j][1]);
    }
  }
}

template <class F, int MAXU_GU, int MAXU_DN, int UPS>
__global__ __launch_bounds__(kW * kWave, 1) void fused_layer_kernel(FusedArgs a) {
  const int G = gridDim.x;
  const int g = blockIdx.x;
  const int w = threadIdx.x / kWave;
  const int lane = lane_id();
  const int B = a.B, k = a.k, E = a.E, D = a.D, Fd = a.Fd;
  const int S = B * k;  // (token, rank) slots
  uint32_t* ctr = reinterpret_cast<uint32_t*>(a.ws + a.L.counters);
  uint32_t tag = ctr[kCtrEpoch] + 1u;  // this call's epoch
  if (tag == 0u) tag = 1u;              // tags start at 1 (the workspace starts zeroed)

  __shared__ int32_t s_idx[kMaxSlots];
  __shared__ float s_gw[kMaxSlots];
  __shared__ ExpertGroup s_grp[kMaxSlots];
  __shared__ int s_U;
  __shared__ int s_timeout;
  __shared__ int s_jx;
  __shared__ __align__(16) uint8_t s_buf[kLdsBytes];

  const int NX = a.nx;
  const int xcd = (int)xcc_id();
  const int GX = G / NX;  // workgroups per XCD
  if (threadIdx.x == 0) {
    s_timeout = 0;
    // Index inside the XCD: every call adds exactly GX to each XCD's counter.
    const uint32_t old = __hip_atomic_fetch_add(ctr + kCtrXcdBase + xcd, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_WORKGROUP);
    s_jx = (int)(old % (uint32_t)GX);
    if (a.trace) {
      a.trace[blockIdx.x * kTracePoints + 8] = (uint64_t)xcd;
      a.trace[blockIdx.x * kTracePoints + 9] = (uint64_t)old;
    }
  }
  stamp(a, 0);

  // ---------------------------------------------------------------- 1. routing
  uint64_t* lg = reinterpret_cast<uint64_t*>(a.ws + a.L.logit_tags);  // [B][E][2]: high, low halves
  for (int e = g; e < E; e += G) {
    const float* row = a.router_w + (int64_t)e * D;
    double acc[kMaxTok];
#pragma unroll
    for (int t = 0; t < kMaxTok; ++t) acc[t] = 0.0;
    for (int c = 4 * (w * kWave + lane); c < D; c += 4 * kWave * kW) {
      const float4 wv = *reinterpret_cast<const float4*>(row + c);
#pragma unroll
      for (int t = 0; t < kMaxTok; ++t) {
        if (t < B) {
          const uint2 xv = *reinterpret_cast<const uint2*>(a.x + (int64_t)t * D + c);
          acc[t] = __builtin_fma((double)wv.x, (double)bf16_to_f32(xv.x & 0xFFFFu), acc[t]);
          acc[t] = __builtin_fma((double)wv.y, (double)bf16_to_f32(xv.x >> 16), acc[t]);
          acc[t] = __builtin_fma((double)wv.z, (double)bf16_to_f32(xv.y & 0xFFFFu), acc[t]);
          acc[t] = __builtin_fma((double)wv.w, (double)bf16_to_f32(xv.y >> 16), acc[t]);
        }
      }
    }
    double* s_part = reinterpret_cast<double*>(s_buf);  // [kW][kMaxTok]
#pragma unroll
    for (int t = 0; t < kMaxTok; ++t) {
      if (t < B) {
        const double v = wave_sum_dpp_f64(acc[t]);
        if (lane == 63) s_part[w * kMaxTok + t] = v;
      }
    }
    __syncthreads();
    if (threadIdx.x < B) {
      const int t = threadIdx.x;
      double s = 0.0;
#pragma unroll
      for (int i = 0; i < kW; ++i) s += s_part[i * kMaxTok + t];
      uint64_t* p = lg + ((int64_t)t * E + e) * 2;
      st_dev(p, tagged((uint32_t)__double2hiint(s), tag));
      st_dev(p + 1, tagged((uint32_t)__double2loint(s), tag));
    }
    __syncthreads();
  }
  stamp(a, 1);

  // Gather every logit (spinning until this call's tags appear), then top-k:
  // wave t handles token t.
  for (int t = w; t < B; t += kW) {
    constexpr int kPer = MOE_MAX_EXPERTS / kWave;
    double v[kPer];
    int id[kPer];
    const uint64_t t0 = wall_clock64();
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      id[i] = lane + kWave * i;
      v[i] = 0.0;
      if (id[i] < E) {
        const uint64_t* p = lg + ((int64_t)t * E + id[i]) * 2;
        uint64_t hw = ld_dev(p), lw = ld_dev(p + 1);
        while (tag_of(hw) != tag || tag_of(lw) != tag) {
          if (wall_clock64() - t0 > kSpinTicks) {
            s_timeout = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
          hw = ld_dev(p);
          lw = ld_dev(p + 1);
        }
        v[i] = __hiloint2double((int)payload_of(hw), (int)payload_of(lw));
      }
    }
    uint32_t taken = 0;
    double my_v = 0.0;  // lane r keeps the rank-r selection
    int my_i = 0;
    for (int r = 0; r < k; ++r) {
      double bv = -__builtin_inf();
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const bool ok = id[i] < E && !((taken >> i) & 1u);
        if (ok && (bi == 0x7FFFFFFF || better(v[i], id[i], bv, bi))) {
          bv = v[i];
          bi = id[i];
        }
      }
      wave_argmax(bv, bi);
      if (lane == r) {
        my_v = bv;
        my_i = bi;
      }
      if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    }
    const double top = __shfl(my_v, 0, kWave);
    const double ex = lane < k ? exp(my_v - top) : 0.0;
    double sum = 0.0;
    for (int r = 0; r < k; ++r) sum += __shfl(ex, r, kWave);
    if (lane < k) {
      s_idx[t * k + lane] = my_i;
      s_gw[t * k + lane] = (float)(ex / sum);
    }
  }
  __syncthreads();
  // Group (token, rank) pairs by expert: experts ascending, tokens ascending.
  if (w == 0) {
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += kWave) {
      const int ex = e0 + lane;
      uint32_t mask = 0;
      int slots[kMaxTok];
#pragma unroll
      for (int t = 0; t < kMaxTok; ++t) {
        slots[t] = 0;
        if (t < B) {
          for (int r = 0; r < k; ++r) {
            if (s_idx[t * k + r] == ex) {
              mask |= 1u << t;
              slots[t] = r;
            }
          }
        }
      }
      const uint64_t used = __ballot(ex < E && mask != 0);
      if (ex < E && mask != 0) {
        const int pos = base + __popcll(used & ((1ull << lane) - 1ull));
        ExpertGroup* gr = &s_grp[pos];
        gr->expert = ex;
        gr->n = __popc(mask);
#pragma unroll
        for (int t = 0; t < kMaxTok; ++t) {
          const int p = __popc(mask & ((1u << t) - 1u));
          if ((mask >> t) & 1u) {
            gr->tok[p] = t;
            gr->slot[p] = slots[t];
          }
        }
        for (int p = __popc(mask); p < kMaxTok; ++p) {
          gr->tok[p] = 0;
          gr->slot[p] = 0;
        }
      }
      base += __popcll(used);
    }
    if (lane == 0) s_U = base;
  }
  __syncthreads();
  const int U = s_U;
  if (g == 0) {
    for (int i = threadIdx.x; i < S; i += blockDim.x) {
      if (a.idx_out) a.idx_out[i] = s_idx[i];
      if (a.gw_out) a.gw_out[i] = s_gw[i];
    }
  }
  stamp(a, 2);

  // ---------------------------------------------------------------- 2. gate / up
  const int jx = s_jx;     // index inside the XCD (s_jx was set before the routing syncs)
  const int FS = Fd / NX;  // d_ff slice of this XCD
  const int f0 = xcd * FS;
  uint64_t* ht = reinterpret_cast<uint64_t*>(a.ws + a.L.h_tags);  // [S][Fd]
  {
    const int UG = F::units(D);
    constexpr int kCh = F::kUnitW / 8;
    // Activations: registers for one token; LDS (chunk-major, so lane reads
    // are consecutive) for several.
    float xr[MAXU_GU][F::kUnitW];
    uint4* xl = reinterpret_cast<uint4*>(s_buf);  // [t][chunk][unit], 8 bf16 each
    if (B == 1) {
#pragma unroll
      for (int j = 0; j < MAXU_GU; ++j) {
        const int u = lane + kWave * j;
        if (u < UG) {
#pragma unroll
          for (int i = 0; i < F::kUnitW; i += 2) {
            const uint32_t p = *reinterpret_cast<const uint32_t*>(a.x + (int64_t)u * F::kUnitW + i);
            xr[j][i] = bf16_to_f32(p & 0xFFFFu);
            xr[j][i + 1] = bf16_to_f32(p >> 16);
          }
        }
      }
    } else {
      for (int i = threadIdx.x; i < B * kCh * UG; i += blockDim.x) {
        const int t = i / (kCh * UG);
        const int rem = i - t * kCh * UG;
        const int u = rem / kCh, c = rem - (rem / kCh) * kCh;
        xl[(t * kCh + c) * UG + u] = *reinterpret_cast<const uint4*>(a.x + (int64_t)t * D + u * F::kUnitW + 8 * c);
      }
      __syncthreads();
    }
    const int RPW = (FS + GX - 1) / GX;  // d_ff rows per workgroup
    for (int r = w; r < RPW; r += kW) {
      const int rl = jx * RPW + r;  // row inside the slice
      if (rl >= FS) break;
      const int row = f0 + rl;
      auto rows_of = [&](int uu, typename F::Row& rg, typename F::Row& ru) {
        const int ex = s_grp[uu].expert;
        const uint16_t* gs = a.gate.scale ? reinterpret_cast<const uint16_t*>(
                                                reinterpret_cast<const uint8_t*>(a.gate.scale) + ex * a.gate.scale_stride)
                                          : nullptr;
        const uint16_t* us = a.up.scale ? reinterpret_cast<const uint16_t*>(
                                              reinterpret_cast<const uint8_t*>(a.up.scale) + ex * a.up.scale_stride)
                                        : nullptr;
        rg = F::row(a.gate.base + ex * a.gate.stride, gs, row, D);
        ru = F::row(a.up.base + ex * a.up.stride, us, row, D);
      };
      typename F::Raw c0[MAXU_GU][2], c1[MAXU_GU][2], c2[MAXU_GU][2];
      {
        typename F::Row rg, ru;
        rows_of(0, rg, ru);
        load_pair<F, MAXU_GU>(rg, ru, UG, lane, c0);
        if (U > 1) {
          rows_of(1, rg, ru);
          load_pair<F, MAXU_GU>(rg, ru, UG, lane, c1);
        }
      }
      for (int uu = 0; uu < U; ++uu) {
        if (uu + 2 < U) {
          typename F::Row rg, ru;
          rows_of(uu + 2, rg, ru);
          load_pair<F, MAXU_GU>(rg, ru, UG, lane, c2);
        }
        const ExpertGroup& gr = s_grp[uu];
        for (int i = 0; i < gr.n; ++i) {
          const int t = gr.tok[i];
          float ag = 0.0f, au = 0.0f;
#pragma unroll
          for (int j = 0; j < MAXU_GU; ++j) {
            const int u = lane + kWave * j;
            if (u < UG) {
              if (B == 1) {
                ag += F::dot(c0[j][0], xr[j]);
                au += F::dot(c0[j][1], xr[j]);
              } else {
                float xs[F::kUnitW];
#pragma unroll
                for (int c = 0; c < kCh; ++c) {
                  const uint4 p = xl[(t * kCh + c) * UG + u];
                  xs[8 * c + 0] = bf16_to_f32(p.x & 0xFFFFu);
                  xs[8 * c + 1] = bf16_to_f32(p.x >> 16);
                  xs[8 * c + 2] = bf16_to_f32(p.y & 0xFFFFu);
                  xs[8 * c + 3] = bf16_to_f32(p.y >> 16);
                  xs[8 * c + 4] = bf16_to_f32(p.z & 0xFFFFu);
                  xs[8 * c + 5] = bf16_to_f32(p.z >> 16);
                  xs[8 * c + 6] = bf16_to_f32(p.w & 0xFFFFu);
                  xs[8 * c + 7] = bf16_to_f32(p.w >> 16);
                }
                ag += F::dot(c0[j][0], xs);
                au += F::dot(c0[j][1], xs);
              }
            }
          }
          ag = wave_sum_dpp(ag);
          au = wave_sum_dpp(au);
          if (lane == 63) {
            const float hv = silu(ag) * au;
            st_dev(ht + (int64_t)(t * k + gr.slot[i]) * Fd + row, tagged(__float_as_uint(hv), tag));
          }
        }
#pragma unroll
        for (int j = 0; j < MAXU_GU; ++j) {
          c0[j][0] = c1[j][0];
          c0[j][1] = c1[j][1];
          c1[j][0] = c2[j][0];
          c1[j][1] = c2[j][1];
        }
      }
    }
  }
  stamp(a, 3);

  // ---------------------------------------------------------------- 3. down (partials over the slice)
  // LDS views: h slice per slot, unit blocks padded by 4 floats (conflict-free
  // float4 reads), then the per-slot row partials.
  constexpr int kHB = F::kUnitW + 4;
  float* sh = reinterpret_cast<float*>(s_buf);  // [S][UPS][kHB]
  float* syp = sh + (size_t)S * UPS * kHB;       // [S][rows of this workgroup]
  const int RPWd = (D + GX - 1) / GX;            // output rows per workgroup
  const int RPV = (RPWd + kW - 1) / kW;          // rows per wave
  const int n0 = jx * RPWd;
  {
    __syncthreads();  // the activation view of s_buf is no longer used
    // Gather this XCD's h slice for every slot (written by the XCD's workgroups).
    const uint64_t t0 = wall_clock64();
    for (int i = threadIdx.x; i < S * FS; i += blockDim.x) {
      const int s = i / FS, f = i - (i / FS) * FS;
      const uint64_t* p = ht + (int64_t)s * Fd + f0 + f;
      uint64_t v = ld_dev(p);
      while (tag_of(v) != tag) {
        if (wall_clock64() - t0 > kSpinTicks) {
          s_timeout = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        v = ld_dev(p);
      }
      sh[(s * UPS + f / F::kUnitW) * kHB + f % F::kUnitW] = __uint_as_float(payload_of(v));
    }
    __syncthreads();
    stamp(a, 4);

    const int UD = RPV * UPS;  // (row, slice-unit) pairs per wave per expert
    const int ub = lane % UPS; // this lane's unit inside the slice row (same for all its pairs)
    auto load_dn = [&](int uu, typename F::Raw (&raw)[MAXU_DN]) {
      const int ex = s_grp[uu].expert;
      const uint16_t* ds = a.down.scale ? reinterpret_cast<const uint16_t*>(
                                              reinterpret_cast<const uint8_t*>(a.down.scale) + ex * a.down.scale_stride)
                                        : nullptr;
#pragma unroll
      for (int j = 0; j < MAXU_DN; ++j) {
        const int v = lane + kWave * j;
        const int rloc = w * RPV + v / UPS;
        if (v < UD && rloc < RPWd && n0 + rloc < D) {
          const typename F::Row row = F::row(a.down.base + ex * a.down.stride, ds, n0 + rloc, Fd);
          F::load(row, xcd * UPS + ub, raw[j]);
        }
      }
    };
    typename F::Raw d0[MAXU_DN], d1[MAXU_DN], d2[MAXU_DN];
    load_dn(0, d0);
    if (U > 1) load_dn(1, d1);
    for (int uu = 0; uu < U; ++uu) {
      if (uu + 2 < U) load_dn(uu + 2, d2);
      const ExpertGroup& gr = s_grp[uu];
      for (int i = 0; i < gr.n; ++i) {
        const int s = gr.tok[i] * k + gr.slot[i];
        const float* hx = sh + (s * UPS + ub) * kHB;
#pragma unroll
        for (int j = 0; j < MAXU_DN; ++j) {
          const int v = lane + kWave * j;
          const int rloc = w * RPV + v / UPS;
          const bool ok = v < UD && rloc < RPWd && n0 + rloc < D;
          float pr = ok ? F::dot(d0[j], hx) : 0.0f;
          pr = group_sum_dpp<UPS>(pr);
          if (ok && ub == 0) syp[s * RPWd + rloc] = pr;
        }
      }
#pragma unroll
      for (int j = 0; j < MAXU_DN; ++j) {
        d0[j] = d1[j];
        d1[j] = d2[j];
      }
    }
    __syncthreads();
    stamp(a, 5);
    // Combine the k ranks in rank order and publish this XCD's partial rows.
    uint64_t* pt = reinterpret_cast<uint64_t*>(a.ws + a.L.part_tags);  // [NX][B][D]
    for (int i = threadIdx.x; i < B * RPWd; i += blockDim.x) {
      const int t = i / RPWd, rl = i - (i / RPWd) * RPWd;
      const int n = n0 + rl;
      if (n < D) {
        float acc = 0.0f;
        for (int j = 0; j < k; ++j) acc = __builtin_fmaf(s_gw[t * k + j], syp[(t * k + j) * RPWd + rl], acc);
        st_dev(pt + ((int64_t)xcd * B + t) * D + n, tagged(__float_as_uint(acc), tag));
      }
    }
  }
  stamp(a, 6);

  // ---------------------------------------------------------------- finish: sum the NX partials
  {
    const uint64_t* pt = reinterpret_cast<const uint64_t*>(a.ws + a.L.part_tags);
    const int RF = (RPWd + NX - 1) / NX;  // rows this workgroup finishes
    const int rf0 = xcd * RF;
    const uint64_t t0 = wall_clock64();
    for (int i = threadIdx.x; i < B * RF; i += blockDim.x) {
      const int t = i / RF, rl = rf0 + (i - (i / RF) * RF);
      const int n = n0 + rl;
      if (rl < RPWd && n < D) {
        float acc = 0.0f;
        for (int x = 0; x < NX; ++x) {
          const uint64_t* p = pt + ((int64_t)x * B + t) * D + n;
          uint64_t v = ld_dev(p);
          while (tag_of(v) != tag) {
            if (wall_clock64() - t0 > kSpinTicks) {
              s_timeout = 1;
              break;
            }
            __builtin_amdgcn_s_sleep(1);
            v = ld_dev(p);
          }
          acc += __uint_as_float(payload_of(v));
        }
        if (a.residual) acc += a.residual[(int64_t)t * D + n];
        a.y[(int64_t)t * D + n] = acc;
      }
    }
  }
  __syncthreads();
  stamp(a, 7);
  if (threadIdx.x == 0) {
    if (s_timeout) __hip_atomic_fetch_or(ctr + kCtrTimeout, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // Every workgroup has read the epoch before workgroup 0 gets here
    // (workgroup 0 consumed the logits of all of them), so advance it.
    if (g == 0) ctr[kCtrEpoch] = tag;
  }
}

template <class F, int MAXU_GU, int MAXU_DN, int UPS>
hipError_t launch_fused_t(const FusedArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((fused_layer_kernel<F, MAXU_GU, MAXU_DN, UPS>), dim3(grid), dim3(kW * kWave), 0, s, a);
  return hipGetLastError();
}

template <class F, int UPS>
hipError_t launch_fused_f(const FusedArgs& a, int grid, int gu_units, int dn_units, hipStream_t s) {
  if (gu_units > kWave) {
    return dn_units > kWave ? launch_fused_t<F, 2, 2, UPS>(a, grid, s) : launch_fused_t<F, 2, 1, UPS>(a, grid, s);
  }
  return dn_units > kWave ? launch_fused_t<F, 1, 2, UPS>(a, grid, s) : launch_fused_t<F, 1, 1, UPS>(a, grid, s);
}

template <class F>
hipError_t launch_fused_ups(const FusedArgs& a, int grid, int gu_units, int dn_units, int ups, hipStream_t s) {
  switch (ups) {
    case 1: return launch_fused_f<F, 1>(a, grid, gu_units, dn_units, s);
    case 2: return launch_fused_f<F, 2>(a, grid, gu_units, dn_units, s);
    case 4: return launch_fused_f<F, 4>(a, grid, gu_units, dn_units, s);
    case 8: return launch_fused_f<F, 8>(a, grid, gu_units, dn_units, s);
    case 16: return launch_fused_f<F, 16>(a, grid, gu_units, dn_units, s);
    default: return hipErrorInvalidValue;
  }
}


// Records each workgroup's XCD.  Its LDS footprint matches the layer
// kernel's, so the placement is the same one-workgroup-per-CU placement.
__global__ __launch_bounds__(kW * kWave, 1) void xcc_map_kernel(uint32_t* out) {
  extern __shared__ uint32_t lds_footprint[];  // sized at launch like the layer kernel's LDS
  if (threadIdx.x == 0) {
    lds_footprint[0] = xcc_id();
    out[blockIdx.x] = lds_footprint[0];
  }
}

}  // namespace

FusedShape fused_shape(int fmt, int B, int k, int D, int F, int grid, int nx) {
  FusedShape sh{};
  sh.ok = false;
  if (grid <= 0 || nx <= 0 || nx > kMaxNX || grid % nx) return sh;
  const int uw = fmt == MOE_FMT_Q2K ? 64 : 32;
  const int gx = grid / nx;
  if (F % (nx * uw)) return sh;  // every XCD's d_ff slice is whole units
  const int ups = F / nx / uw;
  if (ups != 1 && ups != 2 && ups != 4 && ups != 8 && ups != 16) return sh;
  sh.gu_units = D / uw;
  if (D % uw || sh.gu_units > 2 * kWave) return sh;
  const int rpwd = (D + gx - 1) / gx;
  const int rpv = (rpwd + kW - 1) / kW;
  sh.dn_units = rpv * ups;
  if (sh.dn_units > 2 * kWave) return sh;
  sh.ups = ups;
  // LDS: activations (B > 1) during gate/up, then h slices and row partials.
  const size_t act = B > 1 ? (size_t)B * D * 2 : 0;
  const size_t down = (size_t)B * k * ups * (uw + 4) * 4 + (size_t)B * k * rpwd * 4;
  if (act > (size_t)kLdsBytes || down > (size_t)kLdsBytes) return sh;
  sh.ok = true;
  return sh;
}

int fused_grid_size() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static int cached[64] = {0};
  if (dev >= 0 && dev < 64 && cached[dev]) return cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) cached[dev] = cus;
  return cus;
}

namespace {
int& xcd_count_slot(int dev) {
  static int nx[64] = {0};  // per device: 0 unknown, -1 unusable, else the XCD count
  return nx[dev];
}
}  // namespace

int xcd_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  return xcd_count_slot(dev);
}

int probe_xcd_count(uint32_t* scratch, int grid, hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  int& nx = xcd_count_slot(dev);
  if (nx) return nx;
  if (grid <= 0 || grid > 4096) return nx = -1;
  hipLaunchKernelGGL(xcc_map_kernel, dim3(grid), dim3(kW * kWave), kLdsBytes + 8 * 1024, s, scratch);
  uint32_t host[4096];
  if (hipMemcpyAsync(host, scratch, sizeof(uint32_t) * grid, hipMemcpyDeviceToHost, s) != hipSuccess) return -1;
  if (hipStreamSynchronize(s) != hipSuccess) return -1;
  int count[kMaxNX] = {0};
  int n = 0;
  for (int b = 0; b < grid; ++b) {
    const uint32_t x = host[b];
    if (x >= (uint32_t)kMaxNX) return nx = -1;
    ++count[x];
    if ((int)x + 1 > n) n = (int)x + 1;
  }
  // Every XCD must hold the same number of workgroups.
  for (int x = 0; x < n; ++x)
    if (count[x] * n != grid) return nx = -1;
  return nx = n;
}

hipError_t launch_fused_layer(int fmt, const float* router_w, const uint16_t* x, const WeightRef& gate,
                              const WeightRef& up, const WeightRef& down, int E, int D, int Fd, int k, int B,
                              uint8_t* ws, const WsLayout& L, float* y, const float* residual, int32_t* idx_out,
                              float* gw_out, uint64_t* trace, hipStream_t s) {
  FusedArgs a;
  a.router_w = router_w;
  a.x = x;
  a.gate = gate;
  a.up = up;
  a.down = down;
  a.ws = ws;
  a.L = L;
  a.y = y;
  a.residual = residual;
  a.idx_out = idx_out;
  a.gw_out = gw_out;
  a.trace = trace;
  a.E = E;
  a.D = D;
  a.Fd = Fd;
  a.k = k;
  a.B = B;
  a.nx = xcd_count();
  const int grid = fused_grid_size();
  const FusedShape sh = fused_shape(fmt, B, k, D, Fd, grid, a.nx);
  if (!sh.ok) return hipErrorInvalidValue;
  switch (fmt) {
    case MOE_FMT_MXFP4: return launch_fused_ups<MxFmt>(a, grid, sh.gu_units, sh.dn_units, sh.ups, s);
    case MOE_FMT_Q2K: return launch_fused_ups<Q2kFmt>(a, grid, sh.gu_units, sh.dn_units, sh.ups, s);
    case MOE_FMT_INT4G32: return launch_fused_ups<Int4Fmt>(a, grid, sh.gu_units, sh.dn_units, sh.ups, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
