// Internal declarations shared by the HIP translation units of libmoedecode.
// Device helpers for the three weight formats, wave reductions, workspace
// layout and the host-side launch functions each .hip file defines.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_decode.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxTok = MOE_MAX_TOKENS;
constexpr int kMaxTopK = MOE_MAX_TOPK;
constexpr int kMaxSlots = kMaxTok * kMaxTopK;  // (token, rank) pairs per layer call

// ---------------------------------------------------------------- format helpers

// E8M0 scale as fp32: the bit pattern e<<23, with e == 0 mapped to the
// subnormal 2^-127 (0x00400000) and e == 255 giving +inf.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return __uint_as_float(e ? (e << 23) : 0x00400000u);
}

// One MXFP4 block at byte offset `o` of a 4-byte aligned row: the 17 bytes
// lie in the five dwords starting at o & ~3.  Returns the exponent byte and
// the 16 code bytes as four dwords (code byte j in byte j%4 of q[j/4]).
struct MxRaw {
  uint32_t d[5];
  uint32_t sh;  // o & 3
};

__device__ __forceinline__ void mx_load(const uint8_t* __restrict__ row, uint32_t o, MxRaw& r) {
  const uint32_t a = o & ~3u;
  const uint4 v = *reinterpret_cast<const uint4*>(__builtin_assume_aligned(row + a, 4));
  r.d[0] = v.x;
  r.d[1] = v.y;
  r.d[2] = v.z;
  r.d[3] = v.w;
  r.d[4] = *reinterpret_cast<const uint32_t*>(__builtin_assume_aligned(row + a + 16, 4));
  r.sh = o & 3u;
}

// Codes start at byte sh+1 (1..4) of the five-dword window; v_perm selects
// four consecutive bytes of (hi:lo), including the whole `hi` dword when the
// shift is 4.
__device__ __forceinline__ void mx_unpack(const MxRaw& r, uint32_t& e, uint32_t q[4]) {
  e = (r.d[0] >> (8 * r.sh)) & 0xFFu;
  const uint32_t sel = 0x03020100u + (r.sh + 1) * 0x01010101u;
  q[0] = __builtin_amdgcn_perm(r.d[1], r.d[0], sel);
  q[1] = __builtin_amdgcn_perm(r.d[2], r.d[1], sel);
  q[2] = __builtin_amdgcn_perm(r.d[3], r.d[2], sel);
  q[3] = __builtin_amdgcn_perm(r.d[4], r.d[3], sel);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two E2M1 values of code byte `sel` of dword q: .x = low nibble, .y = high
// nibble (gfx950 v_cvt_scalef32_pk_f32_fp4 with scale 1).
#define MOE_FP4X2(q, sel) __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((q), 1.0f, (sel))

// Sum over the 32 weights of one MXFP4 block of E2M1[c_i] * x_i (scale not
// applied).  Element 2j is the high nibble of code byte j.
__device__ __forceinline__ float mx_block_dot(const uint32_t q[4], const float* __restrict__ x32) {
  float acc = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float4 xa = *reinterpret_cast<const float4*>(x32 + 8 * w);
    const float4 xb = *reinterpret_cast<const float4*>(x32 + 8 * w + 4);
    const f32x2 p0 = MOE_FP4X2(q[w], 0);
    const f32x2 p1 = MOE_FP4X2(q[w], 1);
    const f32x2 p2 = MOE_FP4X2(q[w], 2);
    const f32x2 p3 = MOE_FP4X2(q[w], 3);
    acc = __builtin_fmaf(p0.y, xa.x, acc);
    acc = __builtin_fmaf(p0.x, xa.y, acc);
    acc = __builtin_fmaf(p1.y, xa.z, acc);
    acc = __builtin_fmaf(p1.x, xa.w, acc);
    acc = __builtin_fmaf(p2.y, xb.x, acc);
    acc = __builtin_fmaf(p2.x, xb.y, acc);
    acc = __builtin_fmaf(p3.y, xb.z, acc);
    acc = __builtin_fmaf(p3.x, xb.w, acc);
  }
  return acc;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

__device__ __forceinline__ float f16_to_f32(uint32_t h16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

// fp32 -> bfloat16 bits, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int v, int old) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_d(double v) {
  const int lo = dpp_i<CTRL, ROW_MASK>(__double2loint(v), 0);
  const int hi = dpp_i<CTRL, ROW_MASK>(__double2hiint(v), 0);
  return __hiloint2double(hi, lo);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF,
                                                               false));
}

// Sum over the wave in a fixed DPP tree, without LDS round trips; the total
// lands in lane 63.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f<0xB1>(v);        // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);        // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);       // row_half_mirror
  v += dpp_f<0x140>(v);       // row_mirror
  v += dpp_f<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_f<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

// Sum over the wave in a fixed DPP tree; the total lands in lane 63.
__device__ __forceinline__ double wave_sum_dpp_f64(double v) {
  v += dpp_d<0xB1>(v);        // quad_perm [1,0,3,2]
  v += dpp_d<0x4E>(v);        // quad_perm [2,3,0,1]
  v += dpp_d<0x141>(v);       // row_half_mirror
  v += dpp_d<0x140>(v);       // row_mirror
  v += dpp_d<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_d<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

// fp64 -> bfloat16 bits, round to nearest even, without double rounding:
// first to fp32 with round-to-odd (24 >= 8 + 2 bits), then fp32 -> bf16 RNE.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double v) {
  float f = (float)v;
  const double back = (double)f;
  if (back != v && !__builtin_isnan(v)) {
    uint32_t u = __float_as_uint(f);
    if (__builtin_fabs(back) > __builtin_fabs(v)) u -= 1u;  // step toward zero
    u |= 1u;
    f = __uint_as_float(u);
  }
  return f32_to_bf16_rne(f);
}

// ---------------------------------------------------------------- RMSNorm
// x_i = bf16_rne(h_i / sqrt(mean(h^2) + eps)), fp64, for one row h[0..D).
// The sum of squares has one fixed order, shared by the stand-alone norm
// kernel and the single-launch layer (so their activations agree bit for
// bit): the row is cut into 8-element chunks, thread i of 512 takes chunks
// i, i+512, ... and adds their squares with fma in element order, each wave
// sums its 64 lanes with the DPP tree of wave_sum_dpp_f64, and the eight
// wave sums are added as ((w0+w1)+(w2+w3))+((w4+w5)+(w6+w7)).
constexpr int kRmsThreads = 512;
constexpr int kRmsWaves = kRmsThreads / kWave;
static_assert(kRmsWaves == 8, "the wave-sum order below names eight waves");

__device__ __forceinline__ double rms_squares8(const float4& a, const float4& b, double ss) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) ss = __builtin_fma((double)v[j], (double)v[j], ss);
  return ss;
}
__device__ __forceinline__ double rms_total(const double* w) {
  return ((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7]));
}

// The divisor of one row.  `fast` allows the quotient to be formed as
// h * r in fp32 (r = 1/denom rounded to fp32): it needs a finite, positive
// denominator whose reciprocal is a normal fp32 number, which also bounds
// every |h_i / denom| by sqrt(D) (eps >= 0).
struct RmsScale {
  double denom;
  float r;
  bool fast;
};
__device__ __forceinline__ RmsScale rms_scale(double total, int D, double eps) {
  RmsScale s;
  s.denom = sqrt(total / D + eps);
  const double r = 1.0 / s.denom;
  s.r = (float)r;
  s.fast = s.denom > 0.0 && r > 0x1p-125 && r < 0x1p125;  // false for NaN and inf
  return s;
}

// Fast form of bf16_rne(h_j / denom) for eight elements, packed low element
// first.  q = RN32(h * r) lies within 1.5 fp32 ulps of the exact quotient
// (one rounding in r, one in the product; in the subnormal range within one
// ulp), so unless q's low 16 bits sit within 2 of the bf16 rounding midpoint
// 0x8000, q and the exact quotient round to the same bfloat16: q rounded to
// nearest (no tie is possible).  `near` is raised otherwise; the caller then
// takes rms_x8_exact.
typedef float rms_f2 __attribute__((ext_vector_type(2)));
typedef __bf16 rms_b2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 rms_x8_fast(const float4& a, const float4& b, float r, bool& near) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const rms_f2 q = {v[2 * j] * r, v[2 * j + 1] * r};
    near |= (uint16_t)(__float_as_uint(q.x) - 0x7FFEu) <= 4u;
    near |= (uint16_t)(__float_as_uint(q.y) - 0x7FFEu) <= 4u;
    o[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(q, rms_b2));
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}
// bf16_rne of the exact fp64 quotients.
__device__ __forceinline__ uint4 rms_x8_exact(const float4& a, const float4& b, double denom) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = f64_to_bf16_rne((double)v[2 * j] / denom) | (f64_to_bf16_rne((double)v[2 * j + 1] / denom) << 16);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// ---------------------------------------------------------------- workspace

// One unique expert of a layer call and the (token, rank) pairs routed to it,
// tokens ascending.
struct ExpertGroup {
  int32_t expert;
  int32_t n;
  int32_t tok[kMaxTok];
  int32_t slot[kMaxTok];  // rank j of the expert in that token's top-k
  int32_t pad[2];
};
static_assert(sizeof(ExpertGroup) == 80, "group record layout");

// Byte offsets of the regions of a layer workspace (each 256-byte aligned).
struct WsLayout {
  size_t counters;  // uint32[64]: zeroed by moe_workspace_init (see kCtr* slots)
  size_t logits;    // fp64 [B][E]
  size_t idx;       // int32 [B][k]
  size_t gw;        // fp32 [B][k]
  size_t ngroups;   // int32 [1]: number of unique experts U
  size_t groups;    // ExpertGroup [B*k]
  size_t xf;        // fp32 [B][D]: the activation widened from bfloat16
  size_t h;         // fp32 [B][k][F]: SiLU(gate) * up per (token, rank)
  size_t yp;        // fp32 [B][k][D]: down projection per (token, rank)
  // Tagged exchange words of the single-launch layer (payload | epoch << 32):
  size_t logit_tags;  // uint64 [B][E][2]: router logit, high and low halves
  size_t h_tags;      // uint64 [B*k][F]: SiLU(gate) * up
  size_t part_tags;   // uint64 [16][B][D]: per-XCD partial outputs (up to 16 XCDs)
  size_t topo;        // uint32 [4096]: scratch of the placement check
  size_t total;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

inline WsLayout layer_ws_layout(int B, int D, int F, int E, int k) {
  WsLayout L;
  size_t o = 0;
  L.counters = o; o = align256(o + 64 * sizeof(uint32_t));
  L.logits = o;   o = align256(o + (size_t)B * E * sizeof(double));
  L.idx = o;      o = align256(o + (size_t)B * k * sizeof(int32_t));
  L.gw = o;       o = align256(o + (size_t)B * k * sizeof(float));
  L.ngroups = o;  o = align256(o + sizeof(int32_t));
  L.groups = o;   o = align256(o + (size_t)B * k * sizeof(ExpertGroup));
  L.xf = o;       o = align256(o + (size_t)B * D * sizeof(float));
  L.h = o;        o = align256(o + (size_t)B * k * F * sizeof(float));
  L.yp = o;       o = align256(o + (size_t)B * k * D * sizeof(float));
  L.logit_tags = o; o = align256(o + (size_t)B * E * 2 * sizeof(uint64_t));
  L.h_tags = o;     o = align256(o + (size_t)B * k * F * sizeof(uint64_t));
  L.part_tags = o;  o = align256(o + (size_t)16 * B * D * sizeof(uint64_t));
  L.topo = o;       o = align256(o + 4096 * sizeof(uint32_t));
  L.total = o;
  return L;
}

// Counter slots inside the counters region.
enum : int {
  kCtrRoute = 0,     // arrivals in the stand-alone routing kernel (reset by its last workgroup)
  kCtrEpoch = 16,    // number of the last completed single-launch call (tags of a call = epoch + 1)
  kCtrXcdBase = 32,  // [16]: per-XCD arrival counters of the single-launch layer
  kCtrBadIds = 62,   // set if a hash-routed layer met an invalid token id or table row (sticky, like the next)
  kCtrTimeout = 63,  // set if a bounded wait gave up; stays set until the workspace is re-initialised
};

// ---------------------------------------------------------------- hash routing
// A hash-routed layer takes each token's experts from a table indexed by its
// token id instead of from the router's top-k.
struct HashRoute {
  const int32_t* table;  // int32 [vocab][k]; null: learned routing
  const int32_t* ids;    // int32 [B] token ids
  int vocab;
};

// Lane r < k: the rank-r expert of token t.  An id outside [0, vocab) or a
// row with an expert outside [0, E) or a repeated one makes the token use
// experts 0..k-1 and raises `bad` (uniform over the wave).  Every lane of
// the wave must call it.
__device__ __forceinline__ int hash_expert(const HashRoute& h, int t, int E, int k, int lane, bool& bad) {
  int id = h.ids[t];
  const bool bad_id = id < 0 || id >= h.vocab;
  id = bad_id ? 0 : id;
  const int e = lane < k ? h.table[(int64_t)id * k + lane] : 0;
  bool mine = lane < k && (e < 0 || e >= E);
  for (int i = 0; i + 1 < k; ++i) mine |= lane < k && lane > i && e == __builtin_amdgcn_readlane(e, i);
  bad = bad_id || __ballot(mine) != 0ull;
  return bad ? (lane < k ? lane : 0) : e;
}

// ---------------------------------------------------------------- launchers
// Each returns a hipError_t (hipSuccess on success).

struct WeightRef {
  const uint8_t* base;      // MXFP4 / Q2_K blocks or INT4 code words
  const uint16_t* scale;    // INT4 scales (else null)
  int64_t stride;           // bytes between experts
  int64_t scale_stride;     // bytes between experts' scales
  int layout;               // enum moe_layout (gate and up are always MOE_LAYOUT_ROWS)
};

// Block number of block j (32 columns) of row n of an MXFP4 matrix [N][K] in
// MOE_LAYOUT_MFMA16: tile c = j/8, half j/4 % 2, quarter j % 4, 16-row group
// n/16, row n % 16.
__device__ __forceinline__ int64_t mfma16_block(int64_t n, int j, int N) {
  return ((((int64_t)(j >> 3) * (N >> 4) + (n >> 4)) * 2 + ((j >> 2) & 1)) * 4 + (j & 3)) * 16 + (n & 15);
}

// Columns per tile of MOE_LAYOUT_TILE256.
constexpr int kTileCols = 256;

hipError_t launch_gemv(int fmt, const void* w0, const uint16_t* scale, int N, int K, const float* x,
                       int B, float* y, hipStream_t s);

hipError_t launch_route(const float* router_w, int E, int D, const uint16_t* x_bf16, int B, int k,
                        uint8_t* ws, const WsLayout& L, int32_t* idx_out, float* gw_out,
                        double* logits_out, hipStream_t s, const HashRoute& hr = HashRoute{});

hipError_t launch_gate_up(int fmt, const WeightRef& gate, const WeightRef& up, int D, int F, int B,
                          int k, uint8_t* ws, const WsLayout& L, hipStream_t s);

hipError_t launch_down(int fmt, const WeightRef& down, int D, int F, int B, int k, uint8_t* ws,
                       const WsLayout& L, hipStream_t s);

hipError_t launch_combine(int D, int B, int k, const uint8_t* ws, const WsLayout& L, float* y,
                          const float* residual, hipStream_t s);

hipError_t launch_rmsnorm_bf16(const float* h, int B, int D, double eps, uint16_t* out, hipStream_t s);

hipError_t launch_quantize_int4(const uint8_t* mx, int64_t ngroups, int32_t* q, uint16_t* scale,
                                hipStream_t s);

hipError_t launch_validate_mxfp4(const uint8_t* blocks, int64_t n, int32_t* bad, hipStream_t s);

hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t s);

// Pure-read probe (stream.hip): reads [src, src + bytes) with pattern
// (enum moe_stream_pattern), one XOR per workgroup into sink[MOE_STREAM_GRID].
hipError_t launch_stream_read(const void* src, int64_t bytes, int pattern, uint32_t* sink, hipStream_t s);

// dst[(c*N + n)*tile + i] = src[n*tiles*tile + c*tile + i] for c < tiles,
// n < N, i < tile (elements of 2 or 4 bytes).
hipError_t launch_tile_rows(const void* src, void* dst, int64_t N, int tiles, int tile_elems, int elem_bytes,
                            hipStream_t s);
// MXFP4 [N][K/32][17] -> MOE_LAYOUT_MFMA16 (N % 16 == 0, K % 256 == 0).
hipError_t launch_tile_mfma16(const uint8_t* src, uint8_t* dst, int N, int K, hipStream_t s);

// Single-launch layer (routing, gate/up, down and combine in one kernel).
struct FusedShape {
  bool ok;
  bool mfma;  // matrix-core down projection (MXFP4, MOE_LAYOUT_MFMA16)
  int gu_units, dn_units, ups;
};
int fused_grid_size();
// fmt: gate/up format, dfmt: down format (enum moe_format).
FusedShape fused_shape(int fmt, int dfmt, int B, int k, int D, int F, int grid, int nx, int down_layout);
// XCD count of the current device, measured once per device (the probe
// synchronises `s`; scratch needs grid uint32).  xcd_count(): 0 not measured
// yet, -1 placement unsuitable for the single-launch layer, else the count.
int probe_xcd_count(uint32_t* scratch, int grid, hipStream_t s);
int xcd_count();
// x: bf16 activations [B][D]; or, with hn set (x unused), the residual
// stream fp32 [1][D] of one token that the kernel RMS-normalises itself
// (B = 1, D <= 4096, D % 8 == 0, matrix-core layout; hn must not alias y).
hipError_t launch_fused_layer(int fmt, int dfmt, const float* router_w, const uint16_t* x, const float* hn, double eps,
                              const WeightRef& gate, const WeightRef& up, const WeightRef& down, int E, int D, int Fd,
                              int k, int B, uint8_t* ws, const WsLayout& L, float* y, const float* residual,
                              int32_t* idx_out, float* gw_out, uint64_t* trace, hipStream_t s,
                              const HashRoute& hr = HashRoute{}, const float* next_router = nullptr);
constexpr int kFusedNormMaxD = 4096;

// Alternative numerics for the MXFP4 matvec (altnum.hip).
hipError_t launch_q8k_quantize(const float* x, int B, int K, int8_t* q, float* d, hipStream_t s);
hipError_t launch_gemv_q8(const uint8_t* w, int N, int K, const int8_t* q, const float* d, int B, float* y,
                          hipStream_t s);
hipError_t launch_half_lut(uint16_t* out, hipStream_t s);
hipError_t launch_gemv_hlut(const uint8_t* w, int N, int K, const float* x, int B, float* y, hipStream_t s);

}  // namespace moe
