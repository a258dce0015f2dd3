// One MoE layer in a single launch: one 512-thread workgroup per compute
// unit, no grid barriers and no memory fences on the hot path.
//
// Workgroups exchange results through tagged 64-bit words: a 32-bit payload
// plus the call's epoch number.  A consumer spins on the words it needs until
// every tag equals the current epoch, so each dependency waits exactly for
// the data it consumes.  All exchanges use agent-coherent 64-bit accesses
// (workgroup-scope stores are not reliably seen by other compute units of the
// same XCD while the kernel runs).  A workgroup learns its XCD from the
// XCC_ID hardware register.  Its index inside the XCD is blockIdx / NX when
// the host's placement probe saw the round-robin placement (workgroup b on
// XCD b % NX; a workgroup placed otherwise reports a failed wait), else it
// comes from an L2-local counter: with one workgroup per compute unit (the
// LDS footprint allows no more), every XCD holds exactly grid/NX of them,
// whatever order the dispatcher used.
//
//  1. Routing.  Workgroup g computes expert g's router logits for every token
//     (fp64) and publishes them device-wide; in a layer stack at B=1 it first
//     RMS-normalises the residual stream itself.  Every workgroup gathers all
//     logits and derives, identically, each token's top-k (largest first, ties
//     to the lower index) -- or, in a hash-routed layer, reads the token's
//     experts from its table row and only their logits -- the softmax
//     weights and the grouping of (token, rank) pairs by expert.
//  2. Gate/up.  XCD x owns the d_ff slice [x*F/NX, (x+1)*F/NX): its workgroups
//     compute h = SiLU(gate.x) * (up.x) for those rows of every selected
//     expert, keeping the next experts' blocks in flight, and publish h.
//     Gate and up may be in another format than down (template F vs FD).
//  3. Down.  XCD x requests its first experts' down blocks, gathers its own h
//     slice, multiplies every down row's slice-x columns by it (partial sums
//     over d_ff) and publishes the partial outputs device-wide; the output
//     rows are then finished by summing the NX partials in XCD order.  The
//     gate weights enter there: on the matrix-core path they are folded into
//     h, so a token's experts accumulate in its MFMA accumulators (experts
//     ascending); the vector path combines the k ranks in rank order.
//
// A token's arithmetic does not depend on the other tokens in the call (same
// lane mapping, same reduction trees), so B=8 rows equal B=1 results bit for
// bit.  Every wait is bounded (about 0.5 s); on timeout a flag is raised in
// the workspace and the kernel runs to completion.
#pragma once

#include <type_traits>

#include "units.h"

namespace moe {
namespace fused {


constexpr int kW = 8;     // waves per workgroup
constexpr int kMaxNX = 16; // XCDs supported
constexpr int kTracePoints = MOE_TRACE_FIELDS;  // 14 time-stamp slots, then the XCD and the raw XCD counter
static_assert(kTracePoints == 16, "trace record layout");
constexpr uint64_t kSpinTicks = 50000000ull;  // 0.5 s of the 100 MHz wall clock

// ---------------------------------------------------------------- tagged exchange

__device__ __forceinline__ uint64_t tagged(uint32_t payload, uint32_t tag) {
  return ((uint64_t)tag << 32) | payload;
}
__device__ __forceinline__ uint32_t tag_of(uint64_t w) { return (uint32_t)(w >> 32); }
__device__ __forceinline__ uint32_t payload_of(uint64_t w) { return (uint32_t)w; }

// device-wide (agent-coherent)
// A global-memory pointer from its integer value (through an address-space
// cast, so that the compiler keeps its accesses global ones).
template <class T>
__device__ __forceinline__ T* as_global(uint64_t v) {
  return (T*)(__attribute__((address_space(1))) T*)v;
}
__device__ __forceinline__ void st_dev(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// First read of a word written by a workgroup of the same XCD: may be served
// by the XCD's L2 (which that workgroup's agent-coherent store went through)
// or by a line this compute unit cached earlier in the call.  A stale value
// is recognised by its tag and read again with ld_dev.
__device__ __forceinline__ uint64_t ld_xcd(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// ---------------------------------------------------------------- DPP reductions

// (dpp_f and the wave sum wave_sum_dpp are in moe_internal.h.)

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


// (value, index) with "better" = larger value, then lower index.
// LDS words polled by other waves of the workgroup: relaxed workgroup-scope
// atomics, which stay ds_read/ds_write (a volatile access through a generic
// pointer becomes a flat access, which the compiler then waits for together
// with every outstanding global load).  One wave's LDS operations complete in
// issue order, so a reader that sees a count also sees the entries before it.
__device__ __forceinline__ void lds_put(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ int lds_get(int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

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

// Top 32 bits of the order-preserving integer image of a double: a > b
// implies order_key32(a) >= order_key32(b).
__device__ __forceinline__ uint32_t order_key32(double v) {
  const uint32_t hi = (uint32_t)__double2hiint(v);
  return (hi & 0x80000000u) ? ~hi : (hi | 0x80000000u);
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  // lanes without a source read 0, the identity of the unsigned maximum
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// Wave-wide unsigned maximum, returned uniformly.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<0xB1>(v));
  v = max(v, dpp_u<0x4E>(v));
  v = max(v, dpp_u<0x141>(v));
  v = max(v, dpp_u<0x140>(v));
  v = max(v, dpp_u<0x142, 0xA>(v));
  v = max(v, dpp_u<0x143, 0xC>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// One selected expert of a layer call: bit t of `mask` (t < 8) is set when
// token t picked the expert, bits 8+3t .. 10+3t hold its rank in that token's
// top-k.
struct LayerGroup {
  int32_t expert;
  uint32_t mask;
};

struct FusedArgs {
  const float* router_w;
  const uint16_t* x;  // bf16 bits [B][D]; unused when hn is set
  // When set: the residual stream h [1][D] (fp32), normalised in the kernel
  // into x = bf16_rne(h / sqrt(mean(h^2) + eps)) (B = 1, d_model <= 4096).
  const float* hn;
  double eps;
  HashRoute hr;  // table set: hash-routed layer
  // Layer stack: the router weights of the layer that runs next (same E and
  // D), or null.  Workgroup g pulls its row g into L2 while it waits for h.
  const float* next_router;
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
  // Set when the placement probe saw workgroup b run on XCD b % nx: then a
  // workgroup's index inside its XCD is blockIdx.x / nx (a workgroup placed
  // otherwise reports a failed wait).  Otherwise the index comes from an L2
  // atomic counter.
  int rr_mode;
};

__device__ __forceinline__ uint32_t xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xFu;  // HW_REG_XCC_ID bits 3:0
}

// Trace records are kept in LDS (thread 0's stamps) and written out once at
// the end, so a stamp costs no global store (and no wait for one).
__device__ __forceinline__ void stamp(bool traced, uint64_t* rec, int point) {
  if (traced && threadIdx.x == 0) rec[point] = wall_clock64();
}

// Marks every dword of a ring slot as used here, on every path: the wave
// waits for the slot's loads at this point, so the compiler knows that no
// load into the slot is pending when the slot is refilled.
template <class T>
__device__ __forceinline__ void consume(const T& raw) {
  static_assert(sizeof(T) % 4 == 0, "ring slots are dwords");
  const uint32_t* d = reinterpret_cast<const uint32_t*>(&raw);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) asm volatile("" ::"v"(d[i]));
}

// Waits (bounded) until every valid word i < N carries `tag`: v[i] holds the
// first read of word addr(i) and receives the current one.  Each pass
// re-reads all stale words together, so one pass costs one memory round trip
// however many words were stale.
template <int N, class Addr>
__device__ __forceinline__ int await_tags(Addr addr, uint64_t (&v)[N], const bool (&valid)[N], uint32_t tag,
                                          uint64_t t0, int* timeout) {
  static_assert(N <= 32, "stale words are tracked in a 32-bit mask");
  int rereads = 0;  // passes that had to read again (reported by the traced entry point)
#pragma nounroll
  for (;; ++rereads) {
    uint32_t stale = 0u;
#pragma unroll
    for (int i = 0; i < N; ++i) stale |= (valid[i] && tag_of(v[i]) != tag) ? (1u << i) : 0u;
    if (stale == 0u) return rereads;
    if (wall_clock64() - t0 > kSpinTicks) {
      *timeout = 1;
      return rereads;
    }
    __builtin_amdgcn_s_sleep(1);
    uint64_t again[N];  // every word is re-read (all requests first); stale ones take the new value
#pragma unroll
    for (int i = 0; i < N; ++i) again[i] = ld_dev(addr(i));
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = ((stale >> i) & 1u) ? again[i] : v[i];
  }
}

// LDS shared by the phases (activations during gate/up; h slices and row
// partials during down; on the matrix-core path both at once).
constexpr int kLdsBytes = 140 * 1024;
// Experts whose weights a wave has in flight or in use: the loads for expert
// uu + R - 1 are issued before expert uu is computed.  The rings are indexed
// with compile-time constants only (no register copies, which would make the
// wave wait for every load in flight), and every load is issued
// unconditionally (past the last expert, one cached unit for the whole wave)
// so the number of loads between a load and its use is fixed.
template <class F>
struct Rings {  // per format, so a format with more live registers can use shallower rings
  static constexpr int kGU = 4;
  static constexpr int kDN = 7;  // six experts (all of them at B=1) requested ahead
};
template <>
struct Rings<MxFmt> {  // three gate/up items in flight per wave: at the end of gate/up the last items
                       // are spread over more waves (a 4-slot ring was 0.5 us slower at B=1, 1.2 us at B=8)
  static constexpr int kGU = 3;
  static constexpr int kDN = 7;
};
template <>
struct Rings<Int4Fmt> {  // its gate/up unpacking keeps more registers live; three gate/up slots as for
                         // MXFP4 (a 4-slot ring was 1.6 us slower at B=1)
  static constexpr int kGU = 3;
  static constexpr int kDN = 6;
};
constexpr int kSpinBatch = 12;  // tagged words a thread reads before its first wait
// Matrix-core down projection: h enters the MFMA as kHTerms E4M3 terms per
// value, term i scaled by 2^(-kHTermStep * i) relative to term 0, and one
// token takes kHCols of the 16 B columns (its terms, then zero columns).
constexpr int kHTerms = 6;
constexpr int kHTermStep = 4;
constexpr int kHCols = 8;
static_assert(kHTerms <= kHCols && 16 % kHCols == 0, "a token's terms fit its columns");
constexpr int kPrefetchExperts = 1;  // one token: experts whose gate/up rows go to L2 during top-k
constexpr bool kPrefetchDown = true;  // ... and their down rows

// The layer shape of the benchmark workloads (256 experts, top 6, d_model
// 4096, d_ff 2048) on a device of 256 compute units in 8 XCDs: builds with
// FULL = true take these as compile-time constants.
constexpr int kFullE = 256, kFullK = 6, kFullD = 4096, kFullF = 2048, kFullG = 256, kFullNX = 8;

// F: format of gate and up; FD: format of down.  CB: the batch width when it
// is known at compile time (0: given at run time; the in-kernel norm implies
// one token).  FULL: the shape above, known at compile time.
template <class F, int MAXU_GU, int MAXU_DN, int UPS, int DNK, bool NORM, class FD, int CB = NORM ? 1 : 0,
          bool FULL = false>
__global__ __launch_bounds__(kW * kWave, 1) void fused_layer_kernel(FusedArgs a) {
  static_assert(!NORM || CB == 1, "the in-kernel norm is built for one token");
  constexpr int kCh = F::kXDw / 4;  // 16-byte chunks of one unit's staged activations
  constexpr int kRingGU = Rings<F>::kGU;
  constexpr int kRingDN = Rings<FD>::kDN;
  const int g = blockIdx.x;
  const int w = threadIdx.x / kWave;
  const int lane = lane_id();
  // The scalars of the routing phase, requested as one group of scalar loads
  // (one wait) and then held in registers: passing them through an empty asm
  // keeps the compiler from reloading them from the argument buffer later,
  // where each reload would also wait for the epoch load below (scalar loads
  // retire out of order, so a wait for one is a wait for all).
  // (Pointers pass as integers and come back as global-memory pointers, so
  // their loads and stores stay global ones.)
  uint64_t router_i = (uint64_t)a.router_w, x_i = (uint64_t)a.x, h_i = (uint64_t)a.hn, ws_i = (uint64_t)a.ws;
  uint64_t ctr_off = a.L.counters, lg_off = a.L.logit_tags, trace_i = (uint64_t)a.trace;
  int G = gridDim.x, NX = a.nx, E = a.E, D = a.D, Bv = a.B, k = a.k;
  int rr_mode = a.rr_mode;
  asm volatile("" : "+s"(router_i), "+s"(x_i), "+s"(h_i), "+s"(ws_i), "+s"(ctr_off), "+s"(lg_off), "+s"(trace_i),
               "+s"(rr_mode));
  // Full-shape builds take the shape as constants: from the first
  // instruction, except the eight-token matrix-core build, which measured
  // faster with run-time values through the routing and constants from
  // gate/up on.
  constexpr bool kConstAll = FULL && (DNK == 0 || CB == 1), kConstLate = FULL && !kConstAll;
  if constexpr (kConstAll) {
    G = kFullG;
    NX = kFullNX;
    E = kFullE;
    D = kFullD;
    k = kFullK;
  } else {
    asm volatile("" : "+s"(G), "+s"(NX), "+s"(E), "+s"(D), "+s"(Bv), "+s"(k));
  }
  const float* router_w = as_global<const float>(router_i);
  const uint16_t* x_in = as_global<const uint16_t>(x_i);
  const float* h_in = as_global<const float>(h_i);
  uint8_t* ws = as_global<uint8_t>(ws_i);
  const bool traced = trace_i != 0u;
  const int B = CB ? CB : Bv, Fd = FULL ? kFullF : a.Fd;
  int S = B * k;  // (token, rank) slots
  const uint64_t t_start = wall_clock64();  // trace slot 0 (kept in a register until the LDS record is set up)
  // First requests: this thread's 8-element chunk of the workgroup's router
  // row and of the activations (x, or h for the in-kernel norm), issued
  // unconditionally (clamped to a valid row and chunk) before the call's
  // epoch and the XCD counter are requested.
  // At the full shape d_model is 8 x the block size, so every thread has a
  // chunk of its own.  (Left to a run-time test, the compiler keeps a path on
  // which a thread skips its chunk; at the join after the first router dot it
  // must then wait for that path's loads, and on the real path the wait
  // covers the arrival atomic's return.)
  const bool own_chunk = (FULL && kFullD == 8 * kW * kWave) || 8 * (int)threadIdx.x < D;
  const int c8 = min(8 * (int)threadIdx.x, D - 8);
  float4 fha, fhb;       // the in-kernel norm: h chunk (requested before the router row)
  if constexpr (NORM) {
    fha = *reinterpret_cast<const float4*>(h_in + c8);
    fhb = *reinterpret_cast<const float4*>(h_in + c8 + 4);
  }
  const float* frow = router_w + (int64_t)min(g, E - 1) * D + c8;
  const float4 fw0 = *reinterpret_cast<const float4*>(frow);
  const float4 fw1 = *reinterpret_cast<const float4*>(frow + 4);
  uint4 fx[kMaxTok];  // x chunks of every token (rows past B - 1 repeat the last one)
  if constexpr (!NORM) {
#pragma unroll
    for (int t = 0; t < kMaxTok; ++t) fx[t] = *reinterpret_cast<const uint4*>(x_in + (int64_t)min(t, B - 1) * D + c8);
  }
  uint32_t* ctr = reinterpret_cast<uint32_t*>(ws + ctr_off);
  // This call's epoch, read with a scalar load issued after the router and
  // activation loads: a vector load of it measured slower (agent-coherent
  // reads of the counter), and a plain one would make the first use of the
  // tag wait for the x and atomic requests issued after it.  Its value is
  // used from the first publication on (tag_now); the compiler may still
  // wait for it earlier, together with later argument loads.  (Workgroup 0
  // advances the counter only after every workgroup has read it.)
  typedef const __attribute__((address_space(4))) uint32_t ConstU32;
  uint32_t epoch = ((ConstU32*)ctr)[kCtrEpoch];
  uint32_t tag = 0u;
  auto tag_now = [&]() {
    asm volatile("" : "+s"(epoch));
    tag = epoch + 1u;
    if (tag == 0u) tag = 1u;  // tags start at 1 (the workspace starts zeroed)
  };

  __shared__ int32_t s_idx[kMaxSlots];
  __shared__ float s_gw[kMaxSlots];
  __shared__ LayerGroup s_grp[kW][kMaxSlots];  // one group table per wave
  __shared__ uint32_t s_mask[MOE_MAX_EXPERTS];  // per expert: tokens that picked it and at which rank
  __shared__ double s_part[kW][kMaxTok];
  __shared__ double s_rms[kW];  // in-kernel norm: the waves' sums of squares
  __shared__ int s_next;                 // matrix-core path: next token slot to gather
  __shared__ int s_gu_next;              // next gate/up work item
  __shared__ int s_pre[kMaxSlots];       // one token: experts in the order the top-k finds them
  __shared__ int s_pre_n;                // ... and how many are known
  __shared__ int s_timeout;
  __shared__ int s_jx;
  __shared__ uint64_t s_trace[kTracePoints];  // this workgroup's trace record (traced calls)
  __shared__ __align__(16) uint8_t s_buf[kLdsBytes];

  const int xcd = (int)xcc_id();
  int GX = G / NX;  // workgroups per XCD
  // Index inside the XCD: every call adds exactly GX to each XCD's counter.
  // The result is first used after the router logits, so its latency hides
  // behind them.
  uint32_t xcd_arrival = 0;
  int trace_rereads = 0;  // thread 0: re-read passes of the logit (low half) and h (high half) waits
  if (threadIdx.x == 0) s_timeout = 0;
  if (traced && threadIdx.x < kTracePoints) s_trace[threadIdx.x] = 0ull;  // slots a path does not stamp read 0
  // Requested once the first router dot has consumed its loads (its result
  // is needed only after the logits).  Thread 0 alone issues it, so the
  // compiler cannot count it at a wait that follows it: a wait for the router
  // row issued after it becomes a wait for every request, the contended
  // atomic's return included.  take_arrival_after orders it behind the
  // partial sums (an empty asm reading them).
  bool arrival_pending = true;
  auto take_arrival = [&]() {
    if (arrival_pending && threadIdx.x == 0 && !rr_mode)
      xcd_arrival = __hip_atomic_fetch_add(ctr + kCtrXcdBase + xcd, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    arrival_pending = false;
  };
  auto take_arrival_after = [&](const double (&acc)[kMaxTok]) {
#pragma unroll
    for (int t = 0; t < kMaxTok; ++t) asm volatile("" ::"v"(acc[t]));
    take_arrival();
  };
  static_assert(MOE_MAX_EXPERTS <= kW * kWave, "one expert word per thread");
  if (threadIdx.x < MOE_MAX_EXPERTS) s_mask[threadIdx.x] = 0u;
  if (threadIdx.x == 0) {
    s_next = 0;
    s_gu_next = 0;
    s_pre_n = 0;
  }

  int UG = F::units(D);
  uint32_t xraw[2][F::kXRaw];
  // With x given, a workgroup with a router row stages the activations from
  // the chunks it loads for the logits (thread i holds elements 8i..8i+7 of
  // every token; F::stage8 puts them in the staged order with the same bits
  // as F::pack_x), so x is not read a second time.
  const bool early_x = NORM || (D <= 8 * kW * kWave && g < E);
  // (The LDS words cleared above are next used after the logits' barriers.)

  // ---------------------------------------------------------------- 1. routing
  uint64_t* lg = reinterpret_cast<uint64_t*>(ws + lg_off);  // [B][E][2]: high, low halves
  // Router logit partial sums over one 8-element chunk of every token.
  auto dot8 = [&](double (&acc)[kMaxTok], const float4& w0, const float4& w1, const uint4 (&xall)[kMaxTok]) {
#pragma unroll
    for (int t = 0; t < kMaxTok; ++t) {
      if (t < B) {
        const uint4 xv = xall[t];
        acc[t] = __builtin_fma((double)w0.x, (double)bf16_to_f32(xv.x & 0xFFFFu), acc[t]);
        acc[t] = __builtin_fma((double)w0.y, (double)bf16_to_f32(xv.x >> 16), acc[t]);
        acc[t] = __builtin_fma((double)w0.z, (double)bf16_to_f32(xv.y & 0xFFFFu), acc[t]);
        acc[t] = __builtin_fma((double)w0.w, (double)bf16_to_f32(xv.y >> 16), acc[t]);
        acc[t] = __builtin_fma((double)w1.x, (double)bf16_to_f32(xv.z & 0xFFFFu), acc[t]);
        acc[t] = __builtin_fma((double)w1.y, (double)bf16_to_f32(xv.z >> 16), acc[t]);
        acc[t] = __builtin_fma((double)w1.z, (double)bf16_to_f32(xv.w & 0xFFFFu), acc[t]);
        acc[t] = __builtin_fma((double)w1.w, (double)bf16_to_f32(xv.w >> 16), acc[t]);
      }
    }
  };
  // Reduces one router row's partial sums and publishes its logits.
  auto publish_logits = [&](int e, double (&acc)[kMaxTok]) {
#pragma unroll
    for (int t = 0; t < kMaxTok; ++t) {
      if (t < B) {
        const double v = wave_sum_dpp_f64(acc[t]);
        if (lane == 63) s_part[w][t] = v;
      }
    }
    __syncthreads();
    tag_now();
    // The last wave publishes (at B < 8 it gathers no token, so the other
    // waves' reads of the logits do not wait behind these stores).
    if (threadIdx.x >= (kW - 1) * kWave && threadIdx.x < (kW - 1) * kWave + B) {
      const int t = threadIdx.x - (kW - 1) * kWave;
      double s = 0.0;
#pragma unroll
      for (int i = 0; i < kW; ++i) s += s_part[i][t];
      uint64_t* p = lg + ((int64_t)t * E + e) * 2;
      st_dev(p, tagged((uint32_t)__double2hiint(s), tag));
      st_dev(p + 1, tagged((uint32_t)__double2loint(s), tag));
    }
    __syncthreads();
  };
  if constexpr (NORM) {
    // One token (B = 1): its activations are the RMS-normalised residual
    // stream, computed here in the chunk order of rms_total (thread i:
    // elements 8i..8i+7, d_model <= 4096) while the first router row is on
    // its way.  Each thread keeps its chunk for the logits and stages it in
    // LDS for gate/up (F::stage8).
    // The loads are issued unconditionally (clamped to valid rows), h first:
    // the norm then waits for h alone while the router row is in flight.
    const bool mine = own_chunk;  // then c8 = 8 * threadIdx.x
    float4 ha = fha, hb = fhb, w0 = fw0, w1 = fw1;
    if (!mine) ha = hb = make_float4(0.f, 0.f, 0.f, 0.f);
    const double ss = wave_sum_dpp_f64(rms_squares8(ha, hb, 0.0));
    if (lane == kWave - 1) s_rms[w] = ss;
    __syncthreads();
    const RmsScale sc = rms_scale(rms_total(s_rms), D, a.eps);
    bool near = !sc.fast;
    uint4 xn = rms_x8_fast(ha, hb, sc.r, near);
    if (near) xn = rms_x8_exact(ha, hb, sc.denom);  // rare: the exact quotients
    if (mine) F::stage8(xn, threadIdx.x, reinterpret_cast<uint4*>(s_buf), UG);
    uint4 xall[kMaxTok];
#pragma unroll
    for (int t = 0; t < kMaxTok; ++t) xall[t] = xn;
    for (int e = g; e < E; e += G) {
      if (e != g) {
        const float* row = router_w + (int64_t)e * D + c8;
        w0 = *reinterpret_cast<const float4*>(row);
        w1 = *reinterpret_cast<const float4*>(row + 4);
      }
      double acc[kMaxTok];
#pragma unroll
      for (int t = 0; t < kMaxTok; ++t) acc[t] = 0.0;
      if (mine) dot8(acc, w0, w1, xall);
      take_arrival_after(acc);
      publish_logits(e, acc);
    }
  } else {
    uint4 xkeep[kMaxTok];  // this thread's x chunks of the first router row, for the staging
    for (int e = g; e < E; e += G) {
      const float* row = router_w + (int64_t)e * D;
      double acc[kMaxTok];
#pragma unroll
      for (int t = 0; t < kMaxTok; ++t) acc[t] = 0.0;
      auto chunk = [&](const int c) {
        const float4 w0 = *reinterpret_cast<const float4*>(row + c);
        const float4 w1 = *reinterpret_cast<const float4*>(row + c + 4);
        uint4 xall[kMaxTok];  // every token's activations requested before the first use
#pragma unroll
        for (int t = 0; t < kMaxTok; ++t)
          xall[t] = *reinterpret_cast<const uint4*>(x_in + (int64_t)min(t, B - 1) * D + c);
        dot8(acc, w0, w1, xall);
        take_arrival_after(acc);
        if (e == g) {
#pragma unroll
          for (int t = 0; t < kMaxTok; ++t) xkeep[t] = xall[t];
        }
      };
      // One 8-weight chunk per thread in straight-line code when the row
      // fits (d_model <= 4096): no loop header for the compiler to wait at.
      if (D <= 8 * kW * kWave) {
        if (e == g) {  // the chunk requested first
          if (own_chunk) {
            dot8(acc, fw0, fw1, fx);
            take_arrival_after(acc);
#pragma unroll
            for (int t = 0; t < kMaxTok; ++t) xkeep[t] = fx[t];
          }
        } else if (own_chunk) {
          chunk(8 * threadIdx.x);
        }
      } else {
        for (int c = 8 * threadIdx.x; c < D; c += 8 * kW * kWave) chunk(c);
      }
      publish_logits(e, acc);
    }
    if (early_x && own_chunk) {  // after the logits are out: not on their path
#pragma unroll
      for (int t = 0; t < kMaxTok; ++t)
        if (t < B) F::stage8(xkeep[t], threadIdx.x, reinterpret_cast<uint4*>(s_buf) + (size_t)t * kCh * UG, UG);
    }
  }
  take_arrival();  // workgroups without a router row
  tag_now();
  if (traced && threadIdx.x == 0) s_trace[0] = t_start;
  stamp(traced, s_trace, 1);
  // Activations for gate/up of a workgroup that has not staged them above
  // (no router row): requested now, staged in LDS ([t][chunk][unit], so
  // lanes read consecutive chunks) after the routing, which hides their
  // latency.  B * units <= 2 * (kW * kWave) for every shape this kernel accepts.
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = threadIdx.x + q * kW * kWave;
    if (!early_x && i < B * UG) {
      F::load_x(x_in + (int64_t)(i / UG) * D, i - (i / UG) * UG, xraw[q]);  // (never with NORM: staged above)
    }
  }
  stamp(traced, s_trace, 2);

  // Gather every logit (all reads issued before the first wait), then top-k:
  // wave t handles token t.  Each lane sorts its four candidates; every round
  // takes the wave-wide best of the lanes' heads and the owner pops it.
  for (int t = w; t < B; t += kW) {
    double my_v = 0.0;  // lane r keeps the rank-r selection
    int my_i = 0;
    if (a.hr.table) {
      // Hash-routed layer: the token's experts come from its table row, in
      // rank order; only their logits are read from the exchange.
      bool bad;
      my_i = hash_expert(a.hr, t, E, k, lane, bad);
      if (bad && lane == 0)
        __hip_atomic_fetch_or(ctr + kCtrBadIds, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t* p = lg + ((int64_t)t * E + my_i) * 2;
      uint64_t wv[2];
      const bool valid[2] = {lane < k, lane < k};
      wv[0] = lane < k ? ld_dev(p) : 0ull;
      wv[1] = lane < k ? ld_dev(p + 1) : 0ull;
      const int rr = await_tags<2>([&](int j) { return p + j; }, wv, valid, tag, wall_clock64(), &s_timeout);
      if (traced && threadIdx.x == 0) trace_rereads = rr;
      if (t == 0) stamp(traced, s_trace, 3);
      if (lane < k) my_v = __hiloint2double((int)payload_of(wv[0]), (int)payload_of(wv[1]));
      if (B == 1) {  // for the prefetching waves
        if (lane < k) lds_put(&s_pre[lane], my_i);
        __builtin_amdgcn_wave_barrier();
        if (lane == 0) lds_put(&s_pre_n, k);
      }
    } else {
      constexpr int kPer = MOE_MAX_EXPERTS / kWave;
      uint64_t hw[kPer], lw[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int id = lane + kWave * i;
        if (id < E) {
          const uint64_t* p = lg + ((int64_t)t * E + id) * 2;
          hw[i] = ld_dev(p);
          lw[i] = ld_dev(p + 1);
        }
      }
      {
        uint64_t wv[2 * kPer];
        bool valid[2 * kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          wv[2 * i] = hw[i];
          wv[2 * i + 1] = lw[i];
          valid[2 * i] = valid[2 * i + 1] = lane + kWave * i < E;
        }
        const int rr = await_tags<2 * kPer>(
            [&](int j) { return lg + ((int64_t)t * E + lane + kWave * (j >> 1)) * 2 + (j & 1); }, wv, valid, tag,
            wall_clock64(), &s_timeout);
        if (traced && threadIdx.x == 0) trace_rereads = rr;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          hw[i] = wv[2 * i];
          lw[i] = wv[2 * i + 1];
        }
      }
      if (t == 0) stamp(traced, s_trace, 3);
      double v[kPer];
      int id[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        id[i] = lane + kWave * i;
        v[i] = -__builtin_inf();
        if (id[i] < E) {
          v[i] = __hiloint2double((int)payload_of(hw[i]), (int)payload_of(lw[i]));
        } else {
          id[i] = 0x7FFFFFFF;
        }
      }
      auto cswap = [&](int p, int q) {
        if (better(v[q], id[q], v[p], id[p])) {
          const double tv = v[p];
          const int ti = id[p];
          v[p] = v[q];
          id[p] = id[q];
          v[q] = tv;
          id[q] = ti;
        }
      };
      cswap(0, 1);
      cswap(2, 3);
      cswap(0, 2);
      cswap(1, 3);
      cswap(1, 2);
      uint32_t key[4];  // order-preserving keys of the sorted candidates (-0.0 keyed as +0.0)
#pragma unroll
      for (int i = 0; i < 4; ++i) key[i] = order_key32(v[i] + 0.0);
      // Each round: the largest head by the top 32 bits of its order-preserving
      // key (one DPP max); when a single lane holds that key its head is the
      // exact winner, else the tied lanes' heads are compared exactly.  The
      // rounds are unrolled and, apart from that rare tie path, branch-free:
      // the winning lane shifts its sorted list by one (a popped slot gets key
      // 0, below every candidate's).
#pragma unroll
      for (int r = 0; r < kMaxTopK; ++r) {
        if (r >= k) break;
        const uint32_t top_key = wave_max_u32(key[0]);
        const uint64_t tied = __ballot(key[0] == top_key);
        int L = (int)__builtin_ctzll(tied);
        if (__builtin_expect(__popcll(tied) != 1, 0)) {
          double ev = key[0] == top_key ? v[0] : -__builtin_inf();
          int ei = key[0] == top_key ? id[0] : 0x7FFFFFFF;
          wave_argmax(ev, ei);
          L = (int)__builtin_ctzll(__ballot(key[0] == top_key && id[0] == ei));
        }
        const double bv = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v[0]), L),
                                           __builtin_amdgcn_readlane(__double2loint(v[0]), L));
        const int bi = __builtin_amdgcn_readlane(id[0], L);
        my_v = lane == r ? bv : my_v;
        my_i = lane == r ? bi : my_i;
        if (B == 1 && lane == 0) {  // for the prefetching waves
          lds_put(&s_pre[r], min(max(bi, 0), E - 1));
          lds_put(&s_pre_n, r + 1);
        }
        const bool pop = lane == L;  // this lane held the winner
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          key[i] = pop ? key[i + 1] : key[i];
          v[i] = pop ? v[i + 1] : v[i];
          id[i] = pop ? id[i + 1] : id[i];
        }
        key[3] = pop ? 0u : key[3];
        v[3] = pop ? -__builtin_inf() : v[3];
        id[3] = pop ? 0x7FFFFFFF : id[3];
      }
    }
    // Softmax over the k selected logits, summed in rank order, shifted by
    // their maximum (rank 0's logit when they come from the top-k).
    double top = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(my_v), 0),
                                  __builtin_amdgcn_readlane(__double2loint(my_v), 0));
    if (a.hr.table) {
      for (int r = 1; r < k; ++r)
        top = fmax(top, __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(my_v), r),
                                         __builtin_amdgcn_readlane(__double2loint(my_v), r)));
    }
    // The gate weights are fp32 outputs: the exponentials, their rank-order
    // sum and the quotients are taken in fp32 (the fp64 difference rounded
    // once), which keeps them within a few fp32 units of the exact weights.
    const float ex = lane < k ? expf((float)(my_v - top)) : 0.0f;
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r)
      if (r < k) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), r));
    if (lane < k) {
      my_i = min(max(my_i, 0), E - 1);  // NaN logits can leave no valid candidate: stay in bounds
      s_idx[t * k + lane] = my_i;
      s_gw[t * k + lane] = ex / sum;
      // bit t: token t picked the expert; bits 8+3t..10+3t: at rank `lane`
      atomicOr(&s_mask[my_i], (1u << t) | ((uint32_t)lane << (8 + 3 * t)));
    }
  }
  if (threadIdx.x == 0) {  // the arrival counter has long returned by now
    if (rr_mode) {
      if (xcd != g % NX) s_timeout = 1;  // not the placement the probe saw: reported as a failed wait
      s_jx = (g / NX) % GX;
    } else {
      s_jx = (int)(xcd_arrival % (uint32_t)GX);
    }
    if (traced) {
      s_trace[kTracePoints - 2] = (uint64_t)xcd;
      s_trace[kTracePoints - 1] = rr_mode ? (1ull << 63) | (uint64_t)(g / NX) : (uint64_t)xcd_arrival;
    }
  }
  // Stage the activations requested above (their loads have long returned:
  // the logit reads were issued after them).  They are opaque until here, so
  // the compiler cannot hoist their rearrangement into the routing, where it
  // would wait for x.
  if (!early_x) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < F::kXRaw; ++i) asm volatile("" : "+v"(xraw[q][i]));
  }
  uint4* xl = reinterpret_cast<uint4*>(s_buf);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = threadIdx.x + q * kW * kWave;
    if (!early_x && i < B * UG) {
      const int t = i / UG, u = i - (i / UG) * UG;
      uint32_t xs[F::kXDw];
      F::pack_x(xraw[q], xs);
#pragma unroll
      for (int c = 0; c < kCh; ++c)
        xl[(t * kCh + c) * UG + u] = make_uint4(xs[4 * c], xs[4 * c + 1], xs[4 * c + 2], xs[4 * c + 3]);
    }
  }
  // One token: while wave 0 selects the experts, the other waves pull this
  // workgroup's gate/up rows of the first ones into the XCD's L2 (taking the
  // workgroup's likely place in the XCD from its index: a wrong guess only
  // prefetches another workgroup's rows), so the first gate/up loads find
  // them there.  Every lane issues one dword load per expert (lanes with no
  // line of their own read the gate tensor's first dword); the values are
  // only consumed after gate/up, whose waits cover these older loads, so no
  // wave waits for them before the barrier below.
  uint32_t pre_sink[kPrefetchExperts];
#pragma unroll
  for (int r = 0; r < kPrefetchExperts; ++r) pre_sink[r] = 0u;
  {
    if (B == 1 && w >= 1) {
      const int FSp = Fd / NX, RPWp = (FSp + GX - 1) / GX;
      const int fr = xcd * FSp + ((int)(blockIdx.x / NX) % GX) * RPWp;
      const int rows = min(RPWp, xcd * FSp + FSp - fr);
      const int64_t rb = F::row_bytes(D), sb = F::scale_row_bytes(D);  // bytes per row: blocks or codes, scales
      const int64_t nbytes = rows > 0 ? rows * rb : 0, sbytes = rows > 0 ? rows * sb : 0;
      const int lines = (int)((nbytes + 127) / 128), slines = (int)((sbytes + 127) / 128);
      const int p = (int)threadIdx.x - kWave;
      const uint64_t t0 = wall_clock64();
#pragma unroll
      for (int r = 0; r < kPrefetchExperts; ++r) {
        if (r < k && lines > 0) {
          while (lds_get(&s_pre_n) <= r && wall_clock64() - t0 < kSpinTicks)
            __builtin_amdgcn_s_sleep(1);
          const int e = min(max(lds_get(&s_pre[r]), 0), E - 1);  // in bounds even after a timed-out wait
          const uint8_t* q8 = a.gate.base;
          if (p < 2 * lines) {
            const WeightRef& m = p < lines ? a.gate : a.up;
            const int64_t off = min((int64_t)(p < lines ? p : p - lines) * 128, nbytes - 1);
            q8 = m.base + e * m.stride + fr * rb + off;
          } else if (p < 2 * lines + 2 * slines) {  // INT4: the rows' scales
            const int q = p - 2 * lines;
            const WeightRef& m = q < slines ? a.gate : a.up;
            const int64_t off = min((int64_t)(q < slines ? q : q - slines) * 128, sbytes - 1);
            q8 = reinterpret_cast<const uint8_t*>(m.scale) + e * m.scale_stride + fr * sb + off;
          } else if (kPrefetchDown && DNK == 2 && a.down.layout == MOE_LAYOUT_MFMA16 && Fd / NX == 256) {
            // the expert's down blocks of this slice for the workgroup's output
            // rows: one contiguous run in the MOE_LAYOUT_MFMA16 order
            const int RPWdp = (D + GX - 1) / GX;
            const int nd0 = ((int)(blockIdx.x / NX) % GX) * RPWdp;
            const int q = p - 2 * lines - 2 * slines;
            if (RPWdp % 16 == 0 && nd0 + RPWdp <= D && q * 128 < RPWdp * 8 * 17)
              q8 = a.down.base + e * a.down.stride + mfma16_block(nd0, xcd * 8, D) * 17 + q * 128;
          }
          q8 -= reinterpret_cast<uintptr_t>(q8) & 3;  // pointer arithmetic keeps it a global load
          pre_sink[r] = *reinterpret_cast<const uint32_t*>(q8);
        }
      }
    }
  }
  __syncthreads();
  stamp(traced, s_trace, 4);
  // Group (token, rank) pairs by expert, experts ascending: one record per
  // selected expert holding its packed token mask.  Every wave builds the
  // table itself (in its own LDS row, read back by the same wave), so no
  // second barrier is needed.  The group table, one group per lane (U <=
  // kMaxSlots = 64): the rings read an expert or a token mask with
  // v_readlane instead of an LDS round trip.  For the matrix-core down
  // projection, the slots of the group's tokens in ascending token order,
  // one byte each (tokens 0..3 in gsl_lo, 4..7 in gsl_hi).
  static_assert(kMaxSlots <= kWave, "one group per lane");
  int U = 0;
  int g_exp;
  uint32_t g_mask, gsl_lo = 0u, gsl_hi = 0u;  // slot tables: filled after gate/up
  if (B == 1) {  // one token: its k distinct experts, placed in ascending order
    U = k;
    if (lane < k) {
      const int ex = s_idx[lane];
      int pos = 0;
      for (int r = 0; r < k; ++r) pos += s_idx[r] < ex ? 1 : 0;
      s_grp[w][pos] = LayerGroup{ex, 1u | ((uint32_t)lane << 8)};
    }
    __builtin_amdgcn_wave_barrier();
    const LayerGroup gr = s_grp[w][min(lane, U - 1)];
    g_exp = gr.expert;
    g_mask = gr.mask;
  } else {
#pragma unroll
    for (int q = 0; q < MOE_MAX_EXPERTS / kWave; ++q) {
      const int ex = q * kWave + lane;
      const uint32_t mask = ex < E ? s_mask[ex] : 0u;
      const uint64_t used = __ballot(mask != 0u);
      if (mask != 0u) s_grp[w][U + __popcll(used & ((1ull << lane) - 1ull))] = LayerGroup{ex, mask};
      U += __popcll(used);
    }
    __builtin_amdgcn_wave_barrier();
    const LayerGroup gr = s_grp[w][min(lane, U - 1)];
    g_exp = gr.expert;
    g_mask = gr.mask;
  }
  auto fill_slot_tables = [&]() {
    uint32_t m = g_mask & 0xFFu;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = m ? __builtin_ctz(m) : 0;
      const uint32_t sl = m ? (uint32_t)(t * k + (int)((g_mask >> (8 + 3 * t)) & 7u)) : 0u;
      if (i < 4)
        gsl_lo |= sl << (8 * i);
      else
        gsl_hi |= sl << (8 * (i - 4));
      m &= m - 1u;
    }
  };
  auto grp_expert = [&](int uu) { return __builtin_amdgcn_readlane(g_exp, uu); };
  auto grp_mask = [&](int uu) { return (uint32_t)__builtin_amdgcn_readlane((int)g_mask, uu); };
  if (g == 0) {
    for (int i = threadIdx.x; i < S; i += kW * kWave) {
      if (a.idx_out) a.idx_out[i] = s_idx[i];
      if (a.gw_out) a.gw_out[i] = s_gw[i];
    }
  }
  stamp(traced, s_trace, 5);

  if constexpr (kConstLate) {  // the same values, now as constants
    G = kFullG;
    NX = kFullNX;
    E = kFullE;
    D = kFullD;
    k = kFullK;
    GX = kFullG / kFullNX;
    S = B * kFullK;
    UG = F::units(kFullD);
  }
  // ---------------------------------------------------------------- 2. gate / up
  const int jx = s_jx;     // index inside the XCD
  const int FS = Fd / NX;  // d_ff slice of this XCD
  const int f0 = xcd * FS;
  uint64_t* ht = reinterpret_cast<uint64_t*>(a.ws + a.L.h_tags);  // [S][Fd]
  const int RPW = (FS + GX - 1) / GX;  // d_ff rows per workgroup
  // Down projection set-up.  The first experts' down weights are requested
  // now, so they stream together with gate/up and are in registers when h
  // arrives (at B=1 they are all of this workgroup's down weights).
  // LDS views: h slice per slot, unit blocks padded by 4 floats (conflict-free
  // float4 reads; Q2_K keeps its sub-block sums there), then the per-slot row
  // partials.
  constexpr int kHB = FD::kUnitW + 4;
  float* sh = reinterpret_cast<float*>(s_buf);  // [S][UPS][kHB]
  // Vector down in digit-plane form (FD::kDigitH): per (slot, unit) a record
  // of 24 plane dwords and the unit's exponent k, padded to 28 dwords.
  constexpr int kHBD = 28;
  uint32_t* shd = reinterpret_cast<uint32_t*>(s_buf);  // [S][UPS][kHBD]
  const int RPWd = (D + GX - 1) / GX;            // output rows per workgroup
  const int RPV = (RPWd + kW - 1) / kW;          // rows per wave
  const int n0 = jx * RPWd;
  // Matrix-core down projection (MXFP4 in MOE_LAYOUT_MFMA16, DNK > 0): the
  // h slice of every slot becomes the B operand of the 16x16x128 scaled
  // MFMA as kHTerms fp8 (E4M3) terms per value, each term with its own E8M0
  // exponent: h ~ sum_i d_i * 2^(e - 4i - 127), d_i an integer in [-8, 7],
  // one e per 32 values (see gather_batch; the slot's gate weight is folded
  // in).  hb: [S][DNK][4 lane groups][kHTerms terms][32 bytes];
  // hsc: [S][4 * DNK] exponents e.  Both take the LDS of the activations,
  // which are dead once gate/up has ended.  Slot S of hb/hsc is all zeros:
  // lanes without a token (or term) read it.
  constexpr int kHbSlot = DNK * 4 * kHTerms * 32;
  uint8_t* hb = s_buf;
  uint8_t* hsc = hb + (size_t)(S + 1) * kHbSlot;
  float* syp = DNK > 0 ? reinterpret_cast<float*>(hsc + (((size_t)(S + 1) * 4 * DNK + 15) & ~(size_t)15))
               : FD::kDigitH ? reinterpret_cast<float*>(shd + (size_t)S * UPS * kHBD)
                             : sh + (size_t)S * UPS * kHB;  // [S][rows of this workgroup]
  const int UD = RPV * UPS;                      // (row, slice-unit) pairs per wave per expert
  const int ub = lane % UPS;                     // this lane's unit inside the slice row
  // Where this lane's down unit lives: unit xcd*UPS + ub of row n, or, in
  // the tiled layout, unit (xcd*UPS + ub) % UPT of row c*D + n of the
  // [(Fd/256)*D][256] matrix, c = (xcd*UPS + ub) / UPT.
  constexpr int UPT = kTileCols / FD::kUnitW;
  const bool tiled = a.down.layout == MOE_LAYOUT_TILE256;
  const int du_row = xcd * UPS + ub;
  const int dunit = tiled ? du_row % UPT : du_row;
  const int64_t drow0 = tiled ? (int64_t)(du_row / UPT) * D : 0;
  const int dK = tiled ? kTileCols : Fd;
  const uint32_t dsh = (uint32_t)dunit & 3u;
  // Matrix-core lane roles: A row / B and C column mi, lane group mg; the
  // lane's A block for k-step ks is block xcd*UPS + 4ks + mg of row
  // n0 + w*RPV + mi (an MFMA16 block number, so one load covers 1088
  // contiguous bytes at the full shape).
  const int mi = lane & 15, mg = lane >> 4;
  const int drl = w * RPV + mi;
  const bool drow_ok = mi < RPV && drl < RPWd && n0 + drl < D;
  // Every lane's rows and blocks exist (the full layer shape): no masking.
  const bool dn_full = RPV == 16 && RPWd % 16 == 0 && n0 + RPWd <= D && UPS % 4 == 0;
  int dblk[DNK > 0 ? DNK : 1];
  bool dok[DNK > 0 ? DNK : 1];
#pragma unroll
  for (int ks = 0; ks < DNK; ++ks) {
    dok[ks] = drow_ok && 4 * ks + mg < UPS;
    dblk[ks] = dok[ks] ? (int)mfma16_block(n0 + drl, xcd * UPS + 4 * ks + mg, D) : 0;
  }
  constexpr int kDnSlot = DNK > 0 ? DNK : MAXU_DN;
  typename FD::Raw dring[kRingDN][kDnSlot];
  // Matrix-core path: per token pair a and k-step, the accumulated down
  // projection of tokens 2a (columns 0..7) and 2a+1 (columns 8..15) over
  // their groups, experts ascending (the order is the same at every batch
  // width, so a token's rows do not depend on the other tokens).
  typedef float v4f_t __attribute__((ext_vector_type(4)));
  v4f_t tacc[kMaxTok / 2][DNK > 0 ? DNK : 1];
#pragma unroll
  for (int a2 = 0; a2 < kMaxTok / 2; ++a2)
#pragma unroll
    for (int ks = 0; ks < (DNK > 0 ? DNK : 1); ++ks) tacc[a2][ks] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
  // Slots past the last expert load this XCD's first h words instead: the
  // h gather has just read them, so the final waits of the ring are cache
  // hits rather than trips to another XCD's weights.
  const uint8_t* hot = reinterpret_cast<const uint8_t*>(ht + f0);
  auto load_dn = [&](int uu, typename FD::Raw(&dst)[kDnSlot]) {
    const bool live = uu < U;
    const int ex = grp_expert(live ? uu : U - 1);
    if constexpr (DNK > 0) {
      const typename FD::Row all{live ? a.down.base + ex * a.down.stride : hot};
#pragma unroll
      for (int ks = 0; ks < DNK; ++ks) FD::load(all, live ? dblk[ks] : 0, dst[ks]);
    } else {
      const uint16_t* ds = a.down.scale ? reinterpret_cast<const uint16_t*>(
                                              reinterpret_cast<const uint8_t*>(a.down.scale) + ex * a.down.scale_stride)
                                        : nullptr;
#pragma unroll
      for (int j = 0; j < MAXU_DN; ++j) {
        const int v = lane + kWave * j;
        const int rloc = w * RPV + v / UPS;
        const bool ok = live && v < UD && rloc < RPWd && n0 + rloc < D;
        const typename FD::Row rw =
            live ? FD::row(a.down.base + ex * a.down.stride, ds, ok ? drow0 + n0 + rloc : 0, dK)
                 : FD::row(hot, reinterpret_cast<const uint16_t*>(hot), 0, dK);
        FD::load(rw, ok ? dunit : 0, dst[j]);
      }
    }
  };
  // Matrix-core path: once the workgroup's rows of h are out, its waves
  // claim token slots (kGatherBatch at a time), read their
  // h slices (the XCD's d_ff columns) and write them to LDS as the MFMA B
  // operand: four fp8 (E4M3) terms per value under one E8M0 exponent per 32
  // values.  With every group's down weights already in the prologue slots
  // (U <= kRingDN - 1) the down projection is a plain loop over the groups.
  const bool dn_walk = U <= kRingDN - 1;
  // kGatherBatch slots per claim (3; 1 when there are no more slots than
  // waves, so that every slot is converted by a wave of its own).
  auto gather_batch = [&](auto nb) -> bool {  // false once every slot is claimed
    constexpr int kGatherBatch = decltype(nb)::value;
    int i0 = 0;
    if (lane == 0) i0 = atomicAdd(&s_next, kGatherBatch);
    i0 = __builtin_amdgcn_readfirstlane(i0);
    if (i0 >= S) return false;
    const int per_slot = DNK * 32;  // lanes of one slot: 4 values each, zeros past FS
    const bool act = lane < per_slot;
    const int fl = 4 * lane;
    const bool inb = act && fl < FS;
    int sl[kGatherBatch];  // every slot t*k + r of the call is some group's
#pragma unroll
    for (int b = 0; b < kGatherBatch; ++b) sl[b] = min(i0 + b, S - 1);
    auto hp = [&](int q) { return ht + (int64_t)sl[q >> 2] * Fd + f0 + fl + (q & 3); };
    uint64_t v[4 * kGatherBatch];
    bool valid[4 * kGatherBatch];
#pragma unroll
    for (int q = 0; q < 4 * kGatherBatch; ++q) {
      valid[q] = inb && i0 + (q >> 2) < S;
      v[q] = valid[q] ? ld_xcd(hp(q)) : 0ull;
    }
    const int rr = await_tags<4 * kGatherBatch>(hp, v, valid, tag, wall_clock64(), &s_timeout);
    trace_rereads += rr << 16;
#pragma unroll
    for (int b = 0; b < kGatherBatch; ++b) {
      if (i0 + b >= S) break;
      // The slot's gate weight is folded into h here (fp32 product), so the
      // matrix cores add a token's experts into one accumulator.
      const float gws = s_gw[sl[b]];
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = valid[4 * b + i] ? gws * __uint_as_float(payload_of(v[4 * b + i])) : 0.0f;
      // The 8 lanes of a 32-value block agree on its exponent k, which puts
      // the block maximum times 2^k in [2^21, 2^22) (k = 148 - the biased
      // exponent of the maximum, at most 127).  N = rint(h * 2^k) is written
      // in six balanced base-16 digits d_i in [-8, 7] (the digits of
      // N + 0x888888 less 8, two's complement nibbles after XOR 8): term i is
      // d_i, exact in E4M3, under the E8M0 exponent 147 - k - 4i stored as
      // 147 - k (255 for a block holding a non-finite value, which makes
      // every term's scale NaN).  The B values of one column thus span only
      // the binades 2^0 .. 2^3: the scaled MFMA sums products whose exponents
      // lie in such a narrow band exactly, while a B column holding values
      // from all of E4M3's range loses the smallest products.
      // |error| <= 2^-22 * the block maximum.
      float mx = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
      mx = fmaxf(mx, dpp_f<0xB1>(mx));   // quad_perm [1,0,3,2]
      mx = fmaxf(mx, dpp_f<0x4E>(mx));   // quad_perm [2,3,0,1]
      mx = fmaxf(mx, dpp_f<0x141>(mx));  // row_half_mirror: the other quad of the 8
      const int ebm = (int)((__float_as_uint(mx) >> 23) & 0xFFu);
      const int kk = min(148 - ebm, 127);
      uint32_t m[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = (int)__builtin_rintf(__builtin_amdgcn_ldexpf(x[i], kk));  // |n| <= 2^22
        m[i] = (uint32_t)(n + 0x888888) ^ 0x888888u;
      }
      // hb byte q of lane group g, k-step ks, term i holds value 128ks +
      // 64(q/16) + 16g + ((q%16)^1): the E2M1 nibble order pairs weight 2j+1
      // with the lower K position, so values are stored pair-swapped.
      const int r = fl & 127, ks = fl >> 7;
      uint32_t* dst = reinterpret_cast<uint32_t*>(
          hb + (size_t)sl[b] * kHbSlot + ((ks * 4 + ((r & 63) >> 4)) * kHTerms) * 32 + (r >> 6) * 16 + (r & 15));
#pragma unroll
      for (int term = 0; term < kHTerms; ++term) {
        float t[4];  // digit 5 - term of each N (bits 20 - 4 term .. 23 - 4 term), sign-extended
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = (float)(((int)(m[i] << (8 + 4 * term))) >> 28);
        int d = __builtin_amdgcn_cvt_pk_fp8_f32(t[1], t[0], 0, false);
        d = __builtin_amdgcn_cvt_pk_fp8_f32(t[3], t[2], d, true);
        if (act) dst[term * 8] = (uint32_t)d;
      }
      if (act && (lane & 7) == 0) hsc[sl[b] * 4 * DNK + (fl >> 5)] = (uint8_t)(ebm == 255 ? 255 : 147 - kk);
    }
    return true;
  };
  auto compute_dn = [&](int uu, const typename FD::Raw(&src)[kDnSlot]) {
    consume(src);
    const uint32_t mask = grp_mask(uu);
    if constexpr (DNK > 0) {
      typedef int v8i __attribute__((ext_vector_type(8)));
      typedef float v4f __attribute__((ext_vector_type(4)));
      v8i A[DNK];
      int ea[DNK];
#pragma unroll
      for (int ks = 0; ks < DNK; ++ks) {
        uint32_t e, q[4];
        FD::unpack(src[ks], (uint32_t)dblk[ks] & 3u, e, q);
        // Rows or blocks outside the matrix contribute zeros (E2M1 has no
        // NaN, and a unit scale keeps the products finite).
        A[ks] = v8i{(int)(dok[ks] ? q[0] : 0u), (int)(dok[ks] ? q[1] : 0u), (int)(dok[ks] ? q[2] : 0u),
                    (int)(dok[ks] ? q[3] : 0u), 0, 0, 0, 0};
        ea[ks] = dok[ks] ? (int)e : 127;
      }
      // Lane (half hh, column c) takes term c of token 2a + hh when that
      // token picked the group; other lanes read the zero slot S.
      const int c = mi % kHCols;  // the column's term (none past kHTerms)
      const int hh = mi / kHCols;
      const int ct = c < kHTerms ? c : 0;
#pragma unroll
      for (int a2 = 0; a2 < kMaxTok / 2; ++a2) {
        if (2 * a2 >= B) break;
        if (((mask >> (2 * a2)) & 3u) == 0u) continue;  // no token of this pair
        const int t = 2 * a2 + hh;
        const bool tok = ((mask >> t) & 1u) != 0u && c < kHTerms;
        const int sl = tok ? t * k + (int)((mask >> (8 + 3 * t)) & 7u) : S;
#pragma unroll
        for (int ks = 0; ks < DNK; ++ks) {
          const uint4* bp =
              reinterpret_cast<const uint4*>(hb + (size_t)sl * kHbSlot + ((ks * 4 + mg) * kHTerms + ct) * 32);
          const uint4 b0 = bp[0], b1 = bp[1];
          const int hs = hsc[sl * 4 * DNK + 4 * ks + mg];
          const int eb = hs == 255 ? 255 : max(hs - kHTermStep * ct, 0);
          const v8i Bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
          tacc[a2][ks] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[ks], Bv, tacc[a2][ks], 4, 0, 0, ea[ks], 0, eb);
        }
      }
    } else if constexpr (FD::kDigitH) {
      for (uint32_t m = mask & 0xFFu; m != 0u; m &= m - 1u) {  // tokens ascending
        const int t = __builtin_ctz(m);
        const int s = t * k + (int)((mask >> (8 + 3 * t)) & 7u);
        // The lane's rows share one unit of h: its planes and exponent, read once.
        const uint4* rec = reinterpret_cast<const uint4*>(shd + (s * UPS + ub) * kHBD);
        uint32_t pl[24];
#pragma unroll
        for (int c = 0; c < 6; ++c) {
          const uint4 v4 = rec[c];
          pl[4 * c] = v4.x;
          pl[4 * c + 1] = v4.y;
          pl[4 * c + 2] = v4.z;
          pl[4 * c + 3] = v4.w;
        }
        const int ke = (int)rec[6].x;
#pragma unroll
        for (int j = 0; j < MAXU_DN; ++j) {
          const int v = lane + kWave * j;
          const int rloc = w * RPV + v / UPS;
          const bool ok = v < UD && rloc < RPWd && n0 + rloc < D;
          float pr = ok ? FD::dn_dot_digits(src[j], pl, ke) : 0.0f;
          pr = group_sum_dpp<UPS>(pr);
          if (ok && ub == 0) syp[s * RPWd + rloc] = pr;
        }
      }
    } else {
      for (uint32_t m = mask & 0xFFu; m != 0u; m &= m - 1u) {  // tokens ascending
        const int t = __builtin_ctz(m);
        const int s = t * k + (int)((mask >> (8 + 3 * t)) & 7u);
        const float* hx = sh + (s * UPS + ub) * kHB;
        // The lane's rows share one unit of h: read it from LDS once.
        float hreg[kHB];
        if (MAXU_DN > 1) {
#pragma unroll
          for (int c = 0; c < kHB / 4; ++c) {
            const float4 v4 = *reinterpret_cast<const float4*>(hx + 4 * c);
            hreg[4 * c] = v4.x;
            hreg[4 * c + 1] = v4.y;
            hreg[4 * c + 2] = v4.z;
            hreg[4 * c + 3] = v4.w;
          }
        }
        const float* hu = MAXU_DN > 1 ? hreg : hx;
#pragma unroll
        for (int j = 0; j < MAXU_DN; ++j) {
          const int v = lane + kWave * j;
          const int rloc = w * RPV + v / UPS;
          const bool ok = v < UD && rloc < RPWd && n0 + rloc < D;
          float pr = ok ? FD::dn_dot(src[j], dsh, hu) : 0.0f;
          pr = group_sum_dpp<UPS>(pr);
          if (ok && ub == 0) syp[s * RPWd + rloc] = pr;
        }
      }
    }
  };
  // Matrix-core down for prologue slots j0 .. j0 + kDnBatch - 1 in one
  // straight-line block (requires dn_full and groups of at most 4 tokens).
  // Slots past the last group compute on the zero operand and store nothing.
  constexpr int kDnBatch = (Rings<FD>::kDN - 1 + 1) / 2;
  auto down_walk_batch = [&](auto j0c) {
    if constexpr (DNK > 0) {
      constexpr int j0 = decltype(j0c)::value;
      typedef int v8i __attribute__((ext_vector_type(8)));
      typedef float v4f __attribute__((ext_vector_type(4)));
      const int c = mi % kHCols, hh = mi / kHCols;  // B <= 2: token hh in half hh (pair 0)
      const int ct = c < kHTerms ? c : 0;
      v8i A[kDnBatch][DNK], Bv[kDnBatch][DNK];
      int ea[kDnBatch][DNK], eb[kDnBatch][DNK], sl[kDnBatch];
#pragma unroll
      for (int b = 0; b < kDnBatch; ++b) {
        const int j = j0 + b;
        if (j >= kRingDN - 1) continue;
        consume(dring[j]);
        const bool live = j < U;
        const uint32_t mask = grp_mask(live ? j : U - 1);
        const bool tok = live && hh < B && ((mask >> hh) & 1u) != 0u && c < kHTerms;
        sl[b] = tok ? hh * k + (int)((mask >> (8 + 3 * hh)) & 7u) : S;
#pragma unroll
        for (int ks = 0; ks < DNK; ++ks) {
          uint32_t e, q[4];
          FD::unpack(dring[j][ks], (uint32_t)dblk[ks] & 3u, e, q);
          A[b][ks] = v8i{(int)q[0], (int)q[1], (int)q[2], (int)q[3], 0, 0, 0, 0};
          ea[b][ks] = (int)e;
          const uint4* bp =
              reinterpret_cast<const uint4*>(hb + (size_t)sl[b] * kHbSlot + ((ks * 4 + mg) * kHTerms + ct) * 32);
          const uint4 b0 = bp[0], b1 = bp[1];
          Bv[b][ks] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
          const int hs = hsc[sl[b] * 4 * DNK + 4 * ks + mg];
          eb[b][ks] = hs == 255 ? 255 : max(hs - kHTermStep * ct, 0);
        }
      }
#pragma unroll
      for (int b = 0; b < kDnBatch; ++b) {
        const int j = j0 + b;
        if (j >= kRingDN - 1 || j >= U) continue;  // past the last group: its slot holds no weights
#pragma unroll
        for (int ks = 0; ks < DNK; ++ks)
          tacc[0][ks] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[b][ks], Bv[b][ks], tacc[0][ks], 4, 0, 0,
                                                                         ea[b][ks], 0, eb[b][ks]);
      }
    }
  };
  // Gate/up work items are (expert group, row) pairs of this workgroup's
  // rows, in group-table order (experts ascending),
  // handed out by an LDS counter: a wave takes its
  // next item when it requests the item's weights (kRingGU - 1 items ahead),
  // so waves that get their data sooner take more items and all finish
  // together.  A wave's first pass also requests the down prologue between
  // its first gate/up slots, so the gate/up data that the ring waits for
  // first is not queued behind down weights used only after the exchange.
  static_assert(2 * Rings<F>::kGU >= Rings<FD>::kDN - 1, "down prologue fits the first gate/up pass");
  {
    const int NR = max(0, min(RPW, FS - jx * RPW));  // rows of this workgroup
    const int NI = NR * U;
    const float inv_nr = 1.0f / (float)max(NR, 1);
    auto group_of = [&](int it) {  // it / NR for 0 <= it < NI (exact after the correction)
      int q = (int)((float)it * inv_nr);
      q -= q * NR > it ? 1 : 0;
      q += (q + 1) * NR <= it ? 1 : 0;
      return q;
    };
    auto take = [&]() {
      int i = 0;
      if (lane == 0) i = atomicAdd(&s_gu_next, 1);
      return __builtin_amdgcn_readfirstlane(i);
    };
    typename F::Raw ring[kRingGU][2][MAXU_GU];
    int item[kRingGU];  // item in each slot (>= NI: a dead slot)
    auto load_gu = [&](int it, typename F::Raw(&dst)[2][MAXU_GU]) {
      const bool live = it < NI;
      const int uu = live ? group_of(it) : U - 1;
      const int row = f0 + jx * RPW + (live ? it - uu * NR : 0);
      const int ex = grp_expert(uu);
      const uint16_t* gs = a.gate.scale ? reinterpret_cast<const uint16_t*>(
                                              reinterpret_cast<const uint8_t*>(a.gate.scale) + ex * a.gate.scale_stride)
                                        : nullptr;
      const uint16_t* us = a.up.scale ? reinterpret_cast<const uint16_t*>(
                                            reinterpret_cast<const uint8_t*>(a.up.scale) + ex * a.up.scale_stride)
                                      : nullptr;
      const typename F::Row rg = F::row(a.gate.base + ex * a.gate.stride, gs, row, D);
      const typename F::Row ru = F::row(a.up.base + ex * a.up.stride, us, row, D);
#pragma unroll
      for (int j = 0; j < MAXU_GU; ++j) {
        const int u = lane + kWave * j;
        const int ul = (live && u < UG) ? u : 0;
        F::load(rg, ul, dst[0][j]);
        F::load(ru, ul, dst[1][j]);
      }
    };
    auto compute_gu = [&](int it, const typename F::Raw(&src)[2][MAXU_GU]) {
      consume(src);
      const int uu = group_of(it);
      const int row = f0 + jx * RPW + (it - uu * NR);
      const uint32_t mask = grp_mask(uu);
      for (uint32_t m = mask & 0xFFu; m != 0u; m &= m - 1u) {  // tokens ascending
        const int t = __builtin_ctz(m);
        float ag = 0.0f, au = 0.0f;
#pragma unroll
        for (int j = 0; j < MAXU_GU; ++j) {
          const int u = lane + kWave * j;
          if (u < UG) {
            uint32_t xs[F::kXDw];
#pragma unroll
            for (int c = 0; c < kCh; ++c) {
              const uint4 p = xl[(t * kCh + c) * UG + u];
              xs[4 * c] = p.x;
              xs[4 * c + 1] = p.y;
              xs[4 * c + 2] = p.z;
              xs[4 * c + 3] = p.w;
            }
            ag += F::gu_dot(src[0][j], (uint32_t)u & 3u, xs);
            au += F::gu_dot(src[1][j], (uint32_t)u & 3u, xs);
          }
        }
        ag = wave_sum_dpp(ag);
        au = wave_sum_dpp(au);
        // Publish h of this row at once.
        if (lane == 63)
          st_dev(ht + (int64_t)(t * k + (int)((mask >> (8 + 3 * t)) & 7u)) * Fd + row,
                 tagged(__float_as_uint(silu(ag) * au), tag));
      }
    };
#pragma unroll
    for (int j = 0; j < kRingGU - 1; ++j) {
      item[j] = take();
      load_gu(item[j], ring[j]);
      __builtin_amdgcn_sched_barrier(0);  // slots are requested in ring order
    }
    auto pass = [&](auto first) {
#pragma unroll
      for (int j = 0; j < kRingGU; ++j) {
        item[(j + kRingGU - 1) % kRingGU] = take();
        load_gu(item[(j + kRingGU - 1) % kRingGU], ring[(j + kRingGU - 1) % kRingGU]);
        if constexpr (decltype(first)::value) {
          if (2 * j < kRingDN - 1) load_dn(2 * j, dring[2 * j]);
          if (2 * j + 1 < kRingDN - 1) load_dn(2 * j + 1, dring[2 * j + 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (item[j] < NI)
          compute_gu(item[j], ring[j]);
        else
          consume(ring[j]);
      }
    };
    pass(std::true_type{});
    // items are taken in increasing order: once a pass ends on a dead slot,
    // every later slot is dead too
    while (item[kRingGU - 1] < NI) pass(std::false_type{});
  }
  stamp(traced, s_trace, 6);
#pragma unroll
  for (int r = 0; r < kPrefetchExperts; ++r) asm volatile("" ::"v"(pre_sink[r]));  // long since arrived
  fill_slot_tables();
  // Layer stack: while this workgroup waits for the XCD's h slice, its row of
  // the next layer's router goes to L2 (one load per 128-byte line); the
  // next launch has the same grid, so its workgroup g runs on this XCD and
  // finds the row there.  The value is only consumed at the end.
  uint32_t nr_sink = 0u;
  if (a.next_router && g < E && (int)threadIdx.x * 32 < D)
    nr_sink = *reinterpret_cast<const uint32_t*>(a.next_router + (int64_t)g * D + 32 * threadIdx.x);

  // ---------------------------------------------------------------- 3. down (partials over the slice)
  if constexpr (DNK == 0 && FD::kDigitH) {
    __syncthreads();  // the activation view of s_buf is no longer used
    stamp(traced, s_trace, 11);
    // Gather this XCD's h slice for every slot in digit-plane form: eight
    // lanes per (slot, unit) record, four consecutive values each.  The
    // unit's exponent k puts its largest |h| in [2^21, 2^22) (k = 148 - the
    // biased exponent of that maximum), N = rint(h * 2^k), and the digits of
    // N + 0x888888 (base 16, each 0..15) less 8 are the balanced digits
    // d in [-8, 7], which XOR 8 turns into two's complement nibbles.  A lane
    // packs its four values' nibbles per plane into a half-word; lane pairs
    // exchange halves (one DPP swap) so the even lane writes planes 0..2 and
    // the odd lane planes 3..5 of their code word.
    static_assert(FD::kUnitW == 32, "eight lanes of four values per unit");
    constexpr int kR = 3;  // records per lane per pass: all their reads go out before one wait
    const int NU = S * UPS;
    const int q8 = lane & 7;
    const bool odd = (q8 & 1) != 0;
    const uint64_t t0 = wall_clock64();
    for (int r0 = 0; r0 < NU; r0 += kR * kW * 8) {
      auto rid = [&](int r) { return r0 + (r * kW + w) * 8 + (lane >> 3); };
      auto hp = [&](int q) {
        const int id = min(rid(q >> 2), NU - 1);
        const int sl = id / UPS;
        return ht + (int64_t)sl * Fd + f0 + (id - sl * UPS) * 32 + 4 * q8 + (q & 3);
      };
      uint64_t v[4 * kR];
      bool valid[4 * kR];
#pragma unroll
      for (int q = 0; q < 4 * kR; ++q) {
        valid[q] = rid(q >> 2) < NU;
        v[q] = valid[q] ? ld_xcd(hp(q)) : 0ull;
      }
      const int rr = await_tags<4 * kR>(hp, v, valid, tag, t0, &s_timeout);
      trace_rereads += rr << 16;
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        if (r0 + (r * kW + w) * 8 >= NU) break;  // the wave's remaining records do not exist
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = valid[4 * r + i] ? __uint_as_float(payload_of(v[4 * r + i])) : 0.0f;
        float mx = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
        mx = fmaxf(mx, dpp_f<0xB1>(mx));   // quad_perm [1,0,3,2]
        mx = fmaxf(mx, dpp_f<0x4E>(mx));   // quad_perm [2,3,0,1]
        mx = fmaxf(mx, dpp_f<0x141>(mx));  // row_half_mirror: the other quad of the eight lanes
        const int eb = (int)((__float_as_uint(mx) >> 23) & 0xFFu);
        const int kk = 148 - eb;
        uint32_t m[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = (int)__builtin_rintf(__builtin_amdgcn_ldexpf(x[i], kk));  // |n| <= 2^22
          m[i] = (uint32_t)(n + 0x888888) ^ 0x888888u;
        }
        uint32_t hw[6];  // plane p: nibble 5 - p of the four values
#pragma unroll
        for (int pl = 0; pl < 6; ++pl) {
          const int sft = 20 - 4 * pl;
          hw[pl] = ((m[0] >> sft) & 15u) | (((m[1] >> sft) & 15u) << 4) | (((m[2] >> sft) & 15u) << 8) |
                   (((m[3] >> sft) & 15u) << 12);
        }
        const uint32_t send0 = odd ? (hw[0] | (hw[1] << 16)) : (hw[3] | (hw[4] << 16));
        const uint32_t send1 = odd ? hw[2] : hw[5];
        const uint32_t recv0 = (uint32_t)dpp_i<0xB1>((int)send0, 0);
        const uint32_t recv1 = (uint32_t)dpp_i<0xB1>((int)send1, 0);
        const uint32_t o0 = odd ? ((recv0 & 0xFFFFu) | (hw[3] << 16)) : (hw[0] | (recv0 << 16));
        const uint32_t o1 = odd ? ((recv0 >> 16) | (hw[4] << 16)) : (hw[1] | (recv0 & 0xFFFF0000u));
        const uint32_t o2 = odd ? (recv1 | (hw[5] << 16)) : (hw[2] | (recv1 << 16));
        const int id = rid(r);
        if (id < NU) {
          uint32_t* rec = shd + id * kHBD;
          const int pb = odd ? 3 : 0, wd = q8 >> 1;
          rec[4 * pb + wd] = o0;
          rec[4 * (pb + 1) + wd] = o1;
          rec[4 * (pb + 2) + wd] = o2;
          if (q8 == 0) rec[24] = eb == 255 ? (uint32_t)kDigitPoison : (uint32_t)kk;
        }
      }
    }
    stamp(traced, s_trace, 12);
    if (traced && threadIdx.x == 0) s_trace[13] = (uint64_t)trace_rereads;
    __syncthreads();
  } else if constexpr (DNK == 0) {
  __syncthreads();  // the activation view of s_buf is no longer used
  stamp(traced, s_trace, 11);
  {
    // Gather this XCD's h slice for every slot (written by the XCD's workgroups).
    const int g_first = threadIdx.x, g_step = kW * kWave;
    const uint64_t t0 = wall_clock64();
    const int total = S * FS;
    for (int i0 = g_first; i0 < total; i0 += kSpinBatch * g_step) {
      auto hptr = [&](int q) {
        const int i = i0 + q * g_step;
        return ht + (int64_t)(i / FS) * Fd + f0 + (i - (i / FS) * FS);
      };
      uint64_t v[kSpinBatch];
      bool valid[kSpinBatch];
#pragma unroll
      for (int q = 0; q < kSpinBatch; ++q) {
        valid[q] = i0 + q * g_step < total;
        v[q] = valid[q] ? ld_xcd(hptr(q)) : 0ull;
      }
      const int rr = await_tags<kSpinBatch>(hptr, v, valid, tag, t0, &s_timeout);
      trace_rereads += rr << 16;
#pragma unroll
      for (int q = 0; q < kSpinBatch; ++q) {
        const int i = i0 + q * g_step;
        if (valid[q]) {
          const int s = i / FS, f = i - (i / FS) * FS;
          sh[(s * UPS + f / FD::kUnitW) * kHB + f % FD::kUnitW] = __uint_as_float(payload_of(v[q]));
        }
      }
    }
    stamp(traced, s_trace, 12);
    if (traced && threadIdx.x == 0) s_trace[13] = (uint64_t)trace_rereads;
    __syncthreads();
    if (FD::kPrepH) {
      for (int i = threadIdx.x; i < S * UPS; i += kW * kWave) FD::prep_h(sh + i * kHB);
      __syncthreads();
    }
  }
  }
  if constexpr (DNK > 0) {
    __syncthreads();  // every row of this workgroup is published; the activations are dead
    stamp(traced, s_trace, 11);
    // the zero B operand and exponents (slot S), read by lanes without a token or term
    for (int i = threadIdx.x; i < kHbSlot / 16; i += kW * kWave)
      reinterpret_cast<uint4*>(hb + (size_t)S * kHbSlot)[i] = make_uint4(0u, 0u, 0u, 0u);
    if (threadIdx.x < 4 * DNK) hsc[S * 4 * DNK + threadIdx.x] = 0;
    if (S <= kW) {
      while (gather_batch(std::integral_constant<int, 1>{})) {
      }
    } else {
      while (gather_batch(std::integral_constant<int, 3>{})) {
      }
    }
    stamp(traced, s_trace, 12);
    if (traced && threadIdx.x == 0) s_trace[13] = (uint64_t)trace_rereads;
    __syncthreads();
  }
  stamp(traced, s_trace, 7);
  if (DNK > 0 && dn_walk && B <= 16 / kHCols && dn_full) {
    // Every group's down weights are in the prologue slots and every group
    // has at most two tokens (one MFMA pass): the groups are computed in
    // straight-line batches, so their LDS reads and MFMAs overlap.
    down_walk_batch(std::integral_constant<int, 0>{});
    down_walk_batch(std::integral_constant<int, kDnBatch>{});
  } else if (DNK > 0 && dn_walk) {  // every group's down weights are in the prologue slots
#pragma unroll
    for (int j = 0; j < kRingDN - 1; ++j)
      if (j < U) compute_dn(j, dring[j]);
  } else {
    // Waves w and w + kW/2 share a SIMD and have the same fixed down work;
    // the issue arbiter favours the older wave of a pair, which left the
    // younger waves several microseconds behind at eight tokens (and the
    // finish waits for the last rows).  The pair swaps priority every group.
    for (int base = 0; base < U; base += kRingDN) {
#pragma unroll
      for (int j = 0; j < kRingDN; ++j) {
        if (((j + (w >= kW / 2 ? 1 : 0)) & 1) != 0)
          __builtin_amdgcn_s_setprio(1);
        else
          __builtin_amdgcn_s_setprio(0);
        load_dn(base + j + kRingDN - 1, dring[(j + kRingDN - 1) % kRingDN]);
        __builtin_amdgcn_sched_barrier(0);
        if (base + j < U)
          compute_dn(base + j, dring[j]);
        else
          consume(dring[j]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }
  if constexpr (DNK > 0) {
    // Each wave publishes its rows of this XCD's partial output for every
    // token straight from its accumulators (the gate weights are already in
    // h): k-steps in order, then the token's terms (an 8-lane DPP sum).  No
    // workgroup barrier: nothing in LDS is read after this point.
    stamp(traced, s_trace, 8);
    uint64_t* pt = reinterpret_cast<uint64_t*>(a.ws + a.L.part_tags);  // [NX][B][D]
    const int c = mi % kHCols, hh = mi / kHCols;
#pragma unroll
    for (int a2 = 0; a2 < kMaxTok / 2; ++a2) {
      if (2 * a2 >= B) break;
      v4f_t v = tacc[a2][0];
#pragma unroll
      for (int ks = 1; ks < DNK; ++ks) v += tacc[a2][ks];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = group_sum_dpp<kHCols>(v[r]);
      const int t = 2 * a2 + hh;
      if (c == 0 && t < B) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = 4 * mg + r, rloc = w * RPV + rr;
          if (rr < RPV && rloc < RPWd && n0 + rloc < D)
            st_dev(pt + ((int64_t)xcd * B + t) * D + n0 + rloc, tagged(__float_as_uint(v[r]), tag));
        }
      }
    }
  } else {
  __syncthreads();
  stamp(traced, s_trace, 8);
  }
  // Vector path: combine the k ranks in rank order and publish this XCD's
  // partial rows (first half of the waves), while the second half gathers the
  // partials of the rows this workgroup finishes.
  if (DNK == 0 && w < kW / 2) {
    uint64_t* pt = reinterpret_cast<uint64_t*>(a.ws + a.L.part_tags);  // [NX][B][D]
    for (int i = threadIdx.x; i < B * RPWd; i += (kW / 2) * kWave) {
      const int t = i / RPWd, rl = i - (i / RPWd) * RPWd;
      const int n = n0 + rl;
      if (n < D) {
        float acc = 0.0f;
        for (int j = 0; j < k; ++j) acc = __builtin_fmaf(s_gw[t * k + j], syp[(t * k + j) * RPWd + rl], acc);
        st_dev(pt + ((int64_t)xcd * B + t) * D + n, tagged(__float_as_uint(acc), tag));
      }
    }
  }
  stamp(traced, s_trace, 9);

  // ---------------------------------------------------------------- finish: sum the NX partials
  if (w >= kW / 2) {
    const uint64_t* pt = reinterpret_cast<const uint64_t*>(a.ws + a.L.part_tags);
    const int RF = (RPWd + NX - 1) / NX;  // rows this workgroup finishes
    const int rf0 = xcd * RF;
    const uint64_t t0 = wall_clock64();
    for (int i = threadIdx.x - (kW / 2) * kWave; i < B * RF; i += (kW / 2) * kWave) {
      const int t = i / RF, rl = rf0 + (i - (i / RF) * RF);
      const int n = n0 + rl;
      if (rl < RPWd && n < D) {
        auto pptr = [&](int x) { return pt + ((int64_t)x * B + t) * D + n; };
        uint64_t v[kMaxNX];
        bool valid[kMaxNX];
#pragma unroll
        for (int x = 0; x < kMaxNX; ++x) {
          valid[x] = x < NX;
          v[x] = valid[x] ? ld_dev(pptr(x)) : 0ull;
        }
        await_tags<kMaxNX>(pptr, v, valid, tag, t0, &s_timeout);
        float acc = 0.0f;
#pragma unroll
        for (int x = 0; x < kMaxNX; ++x)
          if (x < NX) acc += __uint_as_float(payload_of(v[x]));
        if (a.residual) acc += a.residual[(int64_t)t * D + n];
        a.y[(int64_t)t * D + n] = acc;
      }
    }
  }
  __syncthreads();
  stamp(traced, s_trace, 10);
  if (a.trace && threadIdx.x < kTracePoints) a.trace[blockIdx.x * kTracePoints + threadIdx.x] = s_trace[threadIdx.x];
  if (threadIdx.x == 0) {
    if (s_timeout) __hip_atomic_fetch_or(ctr + kCtrTimeout, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // Every workgroup has read the epoch before workgroup 0 gets here
    // (workgroup 0 consumed the logits of all of them), so advance it.
    if (g == 0) ctr[kCtrEpoch] = tag;
  }
  asm volatile("" ::"v"(nr_sink));  // the next layer's router line, long since arrived
}

__host__ __forceinline__ bool full_shape(const FusedArgs& a, int grid) {
  return a.E == kFullE && a.k == kFullK && a.D == kFullD && a.Fd == kFullF && a.nx == kFullNX && grid == kFullG;
}

template <class F, int MAXU_GU, int MAXU_DN, int UPS, int DNK, bool NORM, class FD, int CB = NORM ? 1 : 0,
          bool FULL = false>
hipError_t launch_fused_t(const FusedArgs& a, int grid, hipStream_t s) {
  if (CB && a.B != CB) return hipErrorInvalidValue;
  if (FULL && !full_shape(a, grid)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fused_layer_kernel<F, MAXU_GU, MAXU_DN, UPS, DNK, NORM, FD, CB, FULL>), dim3(grid),
                     dim3(kW * kWave), 0, s, a);
  return hipGetLastError();
}

// DNK: k-steps of the matrix-core down projection (0: vector path).  NORM
// (the kernel normalises the residual stream itself) exists for the
// matrix-core path only.  FD: format of the down projection.
template <class F, int UPS, int DNK, bool NORM = false, class FD = F>
hipError_t launch_fused_f(const FusedArgs& a, int grid, int gu_units, int dn_units, hipStream_t s) {
  // The benchmark shape: builds with every shape parameter known at compile
  // time, at one and at eight tokens (the in-kernel norm: one token).
  if constexpr (kFullF / kFullNX / FD::kUnitW == UPS) {
    constexpr int kGu = kFullD / F::kUnitW > kWave ? 2 : 1;
    constexpr int kDn = DNK > 0 ? 1 : (16 * UPS > kWave ? 2 : 1);  // 16 output rows per wave
    if (full_shape(a, grid) && gu_units == kFullD / F::kUnitW) {
      if (a.B == 1) return launch_fused_t<F, kGu, kDn, UPS, DNK, NORM, FD, 1, true>(a, grid, s);
      if constexpr (!NORM)
        if (a.B == 8) return launch_fused_t<F, kGu, kDn, UPS, DNK, false, FD, 8, true>(a, grid, s);
    }
  }
  if constexpr (DNK > 0) {
    // the full layer shape (d_model > 2048, eight units per XCD slice) has
    // builds of its own for one and for eight tokens
    if constexpr (!NORM && UPS == 8) {
      if (gu_units > kWave && a.B == 1) return launch_fused_t<F, 2, 1, UPS, DNK, false, FD, 1>(a, grid, s);
      if (gu_units > kWave && a.B == 8) return launch_fused_t<F, 2, 1, UPS, DNK, false, FD, 8>(a, grid, s);
    }
    return gu_units > kWave ? launch_fused_t<F, 2, 1, UPS, DNK, NORM, FD>(a, grid, s)
                            : launch_fused_t<F, 1, 1, UPS, DNK, NORM, FD>(a, grid, s);
  } else {
    static_assert(!NORM, "the in-kernel norm is built for the matrix-core path");
    // one- and eight-token builds of the full layer shape (d_model 4096, one
    // 256-column d_ff slice per XCD: eight 32-wide or four 64-wide down units)
    if constexpr (UPS == 8) {
      if (gu_units > kWave && dn_units > kWave) {
        if (a.B == 1) return launch_fused_t<F, 2, 2, UPS, 0, false, FD, 1>(a, grid, s);
        if (a.B == 8) return launch_fused_t<F, 2, 2, UPS, 0, false, FD, 8>(a, grid, s);
      }
    }
    if constexpr (UPS == 4) {
      if (dn_units <= kWave) {
        if (a.B == 1)
          return gu_units > kWave ? launch_fused_t<F, 2, 1, UPS, 0, false, FD, 1>(a, grid, s)
                                  : launch_fused_t<F, 1, 1, UPS, 0, false, FD, 1>(a, grid, s);
        if (a.B == 8)
          return gu_units > kWave ? launch_fused_t<F, 2, 1, UPS, 0, false, FD, 8>(a, grid, s)
                                  : launch_fused_t<F, 1, 1, UPS, 0, false, FD, 8>(a, grid, s);
      }
    }
    if (gu_units > kWave) {
      return dn_units > kWave ? launch_fused_t<F, 2, 2, UPS, 0, false, FD>(a, grid, s)
                              : launch_fused_t<F, 2, 1, UPS, 0, false, FD>(a, grid, s);
    }
    return dn_units > kWave ? launch_fused_t<F, 1, 2, UPS, 0, false, FD>(a, grid, s)
                            : launch_fused_t<F, 1, 1, UPS, 0, false, FD>(a, grid, s);
  }
}

template <class F, class FD = F>
hipError_t launch_fused_ups(const FusedArgs& a, int grid, int gu_units, int dn_units, int ups, hipStream_t s) {
  switch (ups) {
    case 1: return launch_fused_f<F, 1, 0, false, FD>(a, grid, gu_units, dn_units, s);
    case 2: return launch_fused_f<F, 2, 0, false, FD>(a, grid, gu_units, dn_units, s);
    case 4: return launch_fused_f<F, 4, 0, false, FD>(a, grid, gu_units, dn_units, s);
    case 8: return launch_fused_f<F, 8, 0, false, FD>(a, grid, gu_units, dn_units, s);
    case 16: return launch_fused_f<F, 16, 0, false, FD>(a, grid, gu_units, dn_units, s);
    default: return hipErrorInvalidValue;
  }
}

// MXFP4 with the down projections in MOE_LAYOUT_MFMA16 (d_ff slices of at
// most 256 columns per XCD).
template <bool NORM>
hipError_t launch_fused_mfma(const FusedArgs& a, int grid, int gu_units, int ups, hipStream_t s) {
  switch (ups) {
    case 1: return launch_fused_f<MxFmt, 1, 1, NORM>(a, grid, gu_units, 0, s);
    case 2: return launch_fused_f<MxFmt, 2, 1, NORM>(a, grid, gu_units, 0, s);
    case 4: return launch_fused_f<MxFmt, 4, 1, NORM>(a, grid, gu_units, 0, s);
    case 8: return launch_fused_f<MxFmt, 8, 2, NORM>(a, grid, gu_units, 0, s);
    default: return hipErrorInvalidValue;
  }
}

// One instantiation set per weight format (each in its own translation unit).
hipError_t launch_mx(const FusedArgs& a, int grid, int gu_units, int dn_units, int ups, hipStream_t s);
hipError_t launch_mx_mfma(const FusedArgs& a, int grid, int gu_units, int ups, hipStream_t s);
hipError_t launch_mx_mfma_norm(const FusedArgs& a, int grid, int gu_units, int ups, hipStream_t s);
hipError_t launch_q2k(const FusedArgs& a, int grid, int gu_units, int dn_units, int ups, hipStream_t s);
hipError_t launch_int4(const FusedArgs& a, int grid, int gu_units, int dn_units, int ups, hipStream_t s);
// gate/up in MXFP4 or INT4, down in Q2_K
hipError_t launch_mx_q2k(const FusedArgs& a, int grid, int gu_units, int dn_units, int ups, hipStream_t s);
hipError_t launch_int4_q2k(const FusedArgs& a, int grid, int gu_units, int dn_units, int ups, hipStream_t s);

}  // namespace fused
}  // namespace moe
