// Router: logits in fp64, per-token top-k with softmax, and grouping of the
// (token, rank) pairs by expert so that tokens sharing an expert read its
// weights once.
//
// One wave per expert row computes that expert's logit for every token
// (fp64 accumulation of fp32 weight times bfloat16 activation; both products
// are exact in fp64).  Each workgroup then bumps a counter; the workgroup
// that arrives last reads all logits and does the selection, so the whole
// routing step is a single launch.  The counter is reset by that workgroup,
// leaving the workspace ready for the next call.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouteWaves = 4;

// Larger logit first; equal logits -> lower expert index first.
__device__ __forceinline__ bool better(double va, int ia, double vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ wr, int E, int D,
                                                    const uint16_t* __restrict__ xb, int B, int k,
                                                    uint8_t* __restrict__ ws, WsLayout L,
                                                    int32_t* __restrict__ idx_out, float* __restrict__ gw_out,
                                                    double* __restrict__ logits_out, HashRoute hr) {
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  double* logits = reinterpret_cast<double*>(ws + L.logits);
  const int e = blockIdx.x * kRouteWaves + wave;
  if (e < E) {
    const float* row = wr + (int64_t)e * D;
    double acc[kMaxTok];
#pragma unroll
    for (int t = 0; t < kMaxTok; ++t) acc[t] = 0.0;
    for (int c = 4 * lane; c < D; c += 4 * kWave) {
      const float4 w = *reinterpret_cast<const float4*>(row + c);
#pragma unroll
      for (int t = 0; t < kMaxTok; ++t) {
        if (t < B) {
          const uint2 xv = *reinterpret_cast<const uint2*>(xb + (int64_t)t * D + c);
          acc[t] = __builtin_fma((double)w.x, (double)bf16_to_f32(xv.x & 0xFFFFu), acc[t]);
          acc[t] = __builtin_fma((double)w.y, (double)bf16_to_f32(xv.x >> 16), acc[t]);
          acc[t] = __builtin_fma((double)w.z, (double)bf16_to_f32(xv.y & 0xFFFFu), acc[t]);
          acc[t] = __builtin_fma((double)w.w, (double)bf16_to_f32(xv.y >> 16), acc[t]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kMaxTok; ++t) {
      if (t < B) {
        const double v = wave_sum_f64(acc[t]);
        if (lane == 0) logits[(int64_t)t * E + e] = v;
      }
    }
  }

  // Arrive; the last workgroup continues.
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* ctr = reinterpret_cast<uint32_t*>(ws + L.counters) + kCtrRoute;
    const uint32_t prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == gridDim.x - 1);
    if (s_last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  __shared__ int32_t s_idx[kMaxTok * kMaxTopK];
  __shared__ float s_gw[kMaxTok * kMaxTopK];
  // Top-k per token: one wave per token (tokens wave, wave+4).
  for (int t = wave; t < B; t += kRouteWaves) {
    const double* lt = logits + (int64_t)t * E;
    if (hr.table) {  // hash-routed: the table's experts, weighted by their logits
      bool bad;
      const int my_i = hash_expert(hr, t, E, k, lane, bad);
      if (bad && lane == 0)
        __hip_atomic_fetch_or(reinterpret_cast<uint32_t*>(ws + L.counters) + kCtrBadIds, 1u, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
      const double my_v = lane < k ? lt[my_i] : 0.0;
      double top = -__builtin_inf();  // softmax over the k logits, shifted by their maximum
      for (int r = 0; r < k; ++r) top = fmax(top, __shfl(my_v, r, kWave));
      const double ex = lane < k ? exp(my_v - top) : 0.0;
      double sum = 0.0;
      for (int r = 0; r < k; ++r) sum += __shfl(ex, r, kWave);
      if (lane < k) {
        s_idx[t * k + lane] = my_i;
        s_gw[t * k + lane] = (float)(ex / sum);
      }
      continue;
    }
    constexpr int kPer = MOE_MAX_EXPERTS / kWave;  // 4 logits per lane
    double v[kPer];
    int id[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      id[i] = lane + kWave * i;
      v[i] = id[i] < E ? __builtin_nontemporal_load(lt + id[i]) : 0.0;
    }
    uint32_t taken = 0;  // bit i: this lane's i-th logit already selected
    double my_v = 0.0;   // lane r keeps the rank-r selection
    int my_i = 0;
    for (int r = 0; r < k; ++r) {
      double bv = 0.0;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const bool ok = id[i] < E && !((taken >> i) & 1u);
        if (ok && (bi == 0x7FFFFFFF || better(v[i], id[i], bv, bi))) {
          bv = v[i];
          bi = id[i];
        }
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const double ov = __shfl_xor(bv, m, kWave);
        const int oi = __shfl_xor(bi, m, kWave);
        if (oi != 0x7FFFFFFF && (bi == 0x7FFFFFFF || better(ov, oi, bv, bi))) {
          bv = ov;
          bi = oi;
        }
      }
      if (lane == r) {
        my_v = bv;
        my_i = bi;
      }
      if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    }
    // Softmax over the selected logits (rank 0 is the largest), summed in rank order.
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

  int32_t* idx = reinterpret_cast<int32_t*>(ws + L.idx);
  float* gw = reinterpret_cast<float*>(ws + L.gw);
  for (int i = threadIdx.x; i < B * k; i += blockDim.x) {
    idx[i] = s_idx[i];
    gw[i] = s_gw[i];
    if (idx_out) idx_out[i] = s_idx[i];
    if (gw_out) gw_out[i] = s_gw[i];
  }
  if (logits_out) {
    for (int i = threadIdx.x; i < B * E; i += blockDim.x) logits_out[i] = logits[i];
  }
  // Widen the activation to fp32 for the expert phases.
  float* xf = reinterpret_cast<float*>(ws + L.xf);
  for (int i = threadIdx.x; i < B * D; i += blockDim.x) xf[i] = bf16_to_f32(xb[i]);

  // Group (token, rank) pairs by expert, experts ascending, tokens ascending.
  if (wave == 0) {
    ExpertGroup* groups = reinterpret_cast<ExpertGroup*>(ws + L.groups);
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
        ExpertGroup* gr = &groups[pos];
        gr->expert = ex;
        gr->n = __popc(mask);
#pragma unroll
        for (int t = 0; t < kMaxTok; ++t) {
          const int p = __popc(mask & ((1u << t) - 1u));  // tokens ascending
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
    if (lane == 0) *reinterpret_cast<int32_t*>(ws + L.ngroups) = base;
  }
}

}  // namespace

hipError_t launch_route(const float* router_w, int E, int D, const uint16_t* x_bf16, int B, int k, uint8_t* ws,
                        const WsLayout& L, int32_t* idx_out, float* gw_out, double* logits_out, hipStream_t s,
                        const HashRoute& hr) {
  dim3 grid((E + kRouteWaves - 1) / kRouteWaves);
  hipLaunchKernelGGL(route_kernel, grid, dim3(kRouteWaves * kWave), 0, s, router_w, E, D, x_bf16, B, k, ws, L,
                     idx_out, gw_out, logits_out, hr);
  return hipGetLastError();
}

}  // namespace moe
