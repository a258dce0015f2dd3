// Per-format "units" of a weight row for the matvec kernels: a unit is one
// MXFP4 block (32 weights), one INT4 group (32 weights) or a quarter of a
// Q2_K block (64 weights = 4 sub-blocks of 16).  Each format gives the row
// address, the raw dwords of one unit (loaded with dword-aligned vector
// loads) and dot products of a unit with activations:
//
//   dot(raw, sh, x)      fp32 activations of the unit's weights
//   gu_dot(raw, sh, xs)  bfloat16 activations loaded by load_x and staged by
//                        pack_x (gate/up of the single-launch layer)
//   dn_dot(raw, sh, h)   fp32 activations with per-format extras written by
//                        prep_h (down projection of the single-launch layer)
//
// `sh` is the byte offset of an MXFP4 block inside its five-dword window,
// (17 * u) & 3 == u & 3 for unit u; the other formats ignore it.
#pragma once

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// Two E2M1 values of code byte `sel` of dword q as bfloat16: low half = low
// nibble, high half = high nibble (gfx950 v_cvt_scalef32_pk_bf16_fp4, scale 1).
#define MOE_FP4X2_BF16(q, sel) __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((q), 1.0f, (sel))

// a.lo * b.lo + a.hi * b.hi + c (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(bf16x2 a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, as_bf16x2(b), c, false);
}

// Loads the 16 bytes at p (16-byte aligned) as four dwords.
__device__ __forceinline__ void load_u4(const uint16_t* p, uint32_t* d) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  d[0] = v.x;
  d[1] = v.y;
  d[2] = v.z;
  d[3] = v.w;
}

// Marks a unit of h that holds a non-finite value (digit-plane form).
constexpr int kDigitPoison = 0x7FFFFFFF;

struct MxFmt {
  static constexpr int kUnitW = 32;
  static constexpr int kXDw = 16;  // staged dwords: dword j = x[2j+1] | x[2j] << 16
  struct Row { const uint8_t* p; };
  struct Raw { uint32_t d[5]; };
  static __device__ __forceinline__ Row row(const uint8_t* base, const uint16_t*, int64_t n, int K) {
    return Row{base + n * (int64_t)(K / 32) * 17};
  }
  static __device__ __forceinline__ int units(int K) { return K / 32; }
  // bytes of one row of the block array and of the scale array
  static __device__ __forceinline__ int64_t row_bytes(int K) { return (int64_t)(K / 32) * 17; }
  static __device__ __forceinline__ int64_t scale_row_bytes(int) { return 0; }
  static __device__ __forceinline__ void load(const Row& rw, int u, Raw& raw) {
    MxRaw r;
    mx_load(rw.p, 17u * u, r);
#pragma unroll
    for (int i = 0; i < 5; ++i) raw.d[i] = r.d[i];
  }
  static __device__ __forceinline__ void unpack(const Raw& raw, uint32_t sh, uint32_t& e, uint32_t q[4]) {
    MxRaw r;
#pragma unroll
    for (int i = 0; i < 5; ++i) r.d[i] = raw.d[i];
    r.sh = sh;
    mx_unpack(r, e, q);
  }
  static __device__ __forceinline__ float dot(const Raw& raw, uint32_t sh, const float* __restrict__ x32) {
    uint32_t e, q[4];
    unpack(raw, sh, e, q);
    return e8m0_to_f32(e) * mx_block_dot(q, x32);
  }
  // Activations of unit u as loaded (p[j] = x[2j] | x[2j+1] << 16), then
  // rearranged into the staged order; split so the loads can be issued long
  // before the rearrangement waits for them.
  static constexpr int kXRaw = kUnitW / 2;
  static __device__ __forceinline__ void load_x(const uint16_t* __restrict__ xt, int u, uint32_t (&p)[kXRaw]) {
#pragma unroll
    for (int c = 0; c < kXRaw / 4; ++c) load_u4(xt + kUnitW * u + 8 * c, p + 4 * c);
  }
  static __device__ __forceinline__ void pack_x(const uint32_t (&p)[kXRaw], uint32_t (&xs)[kXDw]) {
#pragma unroll
    for (int j = 0; j < 16; ++j) xs[j] = __builtin_amdgcn_alignbit(p[j], p[j], 16);
  }
  // The same staging from thread i's activations 8i..8i+7 of one token (v,
  // as loaded): chunk i%4 of unit i/4; xt is the token's staged array
  // [kXDw/4][units].  Gives the same bits as pack_x.
  static __device__ __forceinline__ void stage8(const uint4& v, int i, uint4* xt, int UG) {
    xt[(i % 4) * UG + i / 4] =
        make_uint4(__builtin_amdgcn_alignbit(v.x, v.x, 16), __builtin_amdgcn_alignbit(v.y, v.y, 16),
                   __builtin_amdgcn_alignbit(v.z, v.z, 16), __builtin_amdgcn_alignbit(v.w, v.w, 16));
  }
  // Code byte j holds element 2j in its high nibble and 2j+1 in its low one,
  // matching the staged pair order.
  static __device__ __forceinline__ float gu_dot(const Raw& raw, uint32_t sh, const uint32_t (&xs)[kXDw]) {
    uint32_t e, q[4];
    unpack(raw, sh, e, q);
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = dot2_bf16(MOE_FP4X2_BF16(q[w], 0), xs[4 * w + 0], acc);
      acc = dot2_bf16(MOE_FP4X2_BF16(q[w], 1), xs[4 * w + 1], acc);
      acc = dot2_bf16(MOE_FP4X2_BF16(q[w], 2), xs[4 * w + 2], acc);
      acc = dot2_bf16(MOE_FP4X2_BF16(q[w], 3), xs[4 * w + 3], acc);
    }
    return e8m0_to_f32(e) * acc;
  }
  static constexpr bool kPrepH = false;
  static constexpr bool kDigitH = false;
  static __device__ __forceinline__ void prep_h(float*) {}
  static __device__ __forceinline__ float dn_dot(const Raw& raw, uint32_t sh, const float* __restrict__ h) {
    return dot(raw, sh, h);
  }
};

struct Q2kFmt {
  static constexpr int kUnitW = 64;  // a quarter of a 256-weight block: 4 sub-blocks of 16
  // Staged activations, per sub-block s: dword 8s+c (c < 4) = x[16s+4c] |
  // x[16s+4c+2] << 16, dword 8s+4+c = x[16s+4c+1] | x[16s+4c+3] << 16; then
  // the four sub-block sums of x as fp32.
  static constexpr int kXDw = 36;
  struct Row { const uint8_t* p; };
  struct Raw { uint32_t qs[4]; uint32_t sc; uint32_t dd; };
  static __device__ __forceinline__ Row row(const uint8_t* base, const uint16_t*, int64_t n, int K) {
    return Row{base + n * (int64_t)(K / 256) * 84};
  }
  static __device__ __forceinline__ int units(int K) { return K / 64; }
  static __device__ __forceinline__ int64_t row_bytes(int K) { return (int64_t)(K / 256) * 84; }
  static __device__ __forceinline__ int64_t scale_row_bytes(int) { return 0; }
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
  static __device__ __forceinline__ float dot(const Raw& raw, uint32_t, const float* __restrict__ x64) {
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
  static constexpr int kXRaw = kUnitW / 2;
  static __device__ __forceinline__ void load_x(const uint16_t* __restrict__ xt, int u, uint32_t (&p)[kXRaw]) {
#pragma unroll
    for (int c = 0; c < kXRaw / 4; ++c) load_u4(xt + kUnitW * u + 8 * c, p + 4 * c);
  }
  // Sum of the four activations in dwords a, b: (a0 + a1) + (b0 + b1).
  static __device__ __forceinline__ float pair_sum(uint32_t a, uint32_t b) {
    return (bf16_to_f32(a & 0xFFFFu) + bf16_to_f32(a >> 16)) + (bf16_to_f32(b & 0xFFFFu) + bf16_to_f32(b >> 16));
  }
  // A sub-block's sum is (P0 + P1) + (P2 + P3) over its four dword pairs, so
  // that two threads holding eight activations each can form it.
  static __device__ __forceinline__ void pack_x(const uint32_t (&p)[kXRaw], uint32_t (&xs)[kXDw]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float ps[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t a = p[8 * s + 2 * c], b = p[8 * s + 2 * c + 1];
        xs[8 * s + c] = __builtin_amdgcn_perm(b, a, 0x05040100u);      // x[+0] | x[+2] << 16
        xs[8 * s + 4 + c] = __builtin_amdgcn_perm(b, a, 0x07060302u);  // x[+1] | x[+3] << 16
        ps[c] = pair_sum(a, b);
      }
      xs[32 + s] = __float_as_uint((ps[0] + ps[1]) + (ps[2] + ps[3]));
    }
  }
  // The same staging from thread i's activations 8i..8i+7 (v): half h = i%2
  // of sub-block (i%8)/2 of unit i/8.  The two threads of a sub-block are
  // adjacent lanes; their partial sums meet through a DPP swap (x + y and
  // y + x round alike).  Gives the same bits as pack_x.
  static __device__ __forceinline__ void stage8(const uint4& v, int i, uint4* xt, int UG) {
    const int u = i / 8, s = (i % 8) / 2, h = i % 2;
    reinterpret_cast<uint2*>(xt + (2 * s) * UG + u)[h] =
        make_uint2(__builtin_amdgcn_perm(v.y, v.x, 0x05040100u), __builtin_amdgcn_perm(v.w, v.z, 0x05040100u));
    reinterpret_cast<uint2*>(xt + (2 * s + 1) * UG + u)[h] =
        make_uint2(__builtin_amdgcn_perm(v.y, v.x, 0x07060302u), __builtin_amdgcn_perm(v.w, v.z, 0x07060302u));
    const float q = pair_sum(v.x, v.y) + pair_sum(v.z, v.w);
    const float sum = q + __int_as_float(dpp_i<0xB1>(__float_as_int(q), 0));  // quad_perm [1,0,3,2]
    if (h == 0) reinterpret_cast<uint32_t*>(xt + 8 * UG + u)[s] = __float_as_uint(sum);
  }
  // The 2-bit codes 0..3 equal twice the E2M1 values of nibbles 0..3, so each
  // code is moved into a nibble and widened by the FP4 conversion; the factor
  // 2 goes into the sub-block scale (exact).
  static __device__ __forceinline__ float gu_dot(const Raw& raw, uint32_t, const uint32_t (&xs)[kXDw]) {
    const float d2 = 2.0f * f16_to_f32(raw.dd & 0xFFFFu);
    const float dmin = f16_to_f32(raw.dd >> 16);
    float acc = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t n0 = raw.qs[s] & 0x33333333u;         // codes m = 0 (low nibble), 2 (high nibble)
      const uint32_t n1 = (raw.qs[s] >> 2) & 0x33333333u;  // codes m = 1, 3
      float sqx = 0.0f;
      sqx = dot2_bf16(MOE_FP4X2_BF16(n0, 0), xs[8 * s + 0], sqx);
      sqx = dot2_bf16(MOE_FP4X2_BF16(n0, 1), xs[8 * s + 1], sqx);
      sqx = dot2_bf16(MOE_FP4X2_BF16(n0, 2), xs[8 * s + 2], sqx);
      sqx = dot2_bf16(MOE_FP4X2_BF16(n0, 3), xs[8 * s + 3], sqx);
      sqx = dot2_bf16(MOE_FP4X2_BF16(n1, 0), xs[8 * s + 4], sqx);
      sqx = dot2_bf16(MOE_FP4X2_BF16(n1, 1), xs[8 * s + 5], sqx);
      sqx = dot2_bf16(MOE_FP4X2_BF16(n1, 2), xs[8 * s + 6], sqx);
      sqx = dot2_bf16(MOE_FP4X2_BF16(n1, 3), xs[8 * s + 7], sqx);
      const uint32_t sb = (raw.sc >> (8 * s)) & 0xFFu;
      acc = __builtin_fmaf(d2 * (float)(sb & 0xFu), sqx, acc);
      acc = __builtin_fmaf(-(dmin * (float)(sb >> 4)), __uint_as_float(xs[32 + s]), acc);
    }
    return acc;
  }
  // Sub-block sums of one unit's h (64 values) into h[64..67].
  static constexpr bool kPrepH = true;
  static constexpr bool kDigitH = false;
  static __device__ __forceinline__ void prep_h(float* h) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float sum = 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 v = *reinterpret_cast<const float4*>(h + 16 * s + 4 * c);
        sum += (v.x + v.y) + (v.z + v.w);
      }
      h[64 + s] = sum;
    }
  }
  static __device__ __forceinline__ float dn_dot(const Raw& raw, uint32_t, const float* __restrict__ h) {
    const float d2 = 2.0f * f16_to_f32(raw.dd & 0xFFFFu);
    const float dmin = f16_to_f32(raw.dd >> 16);
    float acc = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t n0 = raw.qs[s] & 0x33333333u;
      const uint32_t n1 = (raw.qs[s] >> 2) & 0x33333333u;
      float sqx = 0.0f;
      // Byte c of n0 holds the (halved) codes of weights 4c (low nibble) and
      // 4c+2; byte c of n1 those of weights 4c+1 and 4c+3.
#define MOE_Q2K_DN_STEP(c)                                                      \
  {                                                                             \
    const float4 hv = *reinterpret_cast<const float4*>(h + 16 * s + 4 * (c));  \
    const f32x2 a = MOE_FP4X2(n0, c);                                           \
    const f32x2 b = MOE_FP4X2(n1, c);                                           \
    sqx = __builtin_fmaf(a.x, hv.x, sqx);                                       \
    sqx = __builtin_fmaf(b.x, hv.y, sqx);                                       \
    sqx = __builtin_fmaf(a.y, hv.z, sqx);                                       \
    sqx = __builtin_fmaf(b.y, hv.w, sqx);                                       \
  }
      MOE_Q2K_DN_STEP(0)
      MOE_Q2K_DN_STEP(1)
      MOE_Q2K_DN_STEP(2)
      MOE_Q2K_DN_STEP(3)
#undef MOE_Q2K_DN_STEP
      const uint32_t sb = (raw.sc >> (8 * s)) & 0xFFu;
      acc = __builtin_fmaf(d2 * (float)(sb & 0xFu), sqx, acc);
      acc = __builtin_fmaf(-(dmin * (float)(sb >> 4)), h[64 + s], acc);
    }
    return acc;
  }
};

// Offset-binary INT4 codes u = c + 8 (0..15) placed in bytes are FP8 E4M3
// values u * 2^-9 exactly (subnormals continue linearly into the first
// binade), so the FP8 conversions widen eight codes with four instructions;
// the factor 2^9 and the offset 8 are applied once per unit.
#define MOE_FP8X2_BF16(q, hiword) __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((q), 1.0f, (hiword))
#define MOE_FP8X2_F32(q, hiword) __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((q), 1.0f, (hiword))

struct Int4Fmt {
  static constexpr int kUnitW = 32;
  // Staged activations, per code word w (elements 8w..8w+7): dwords 4w..4w+3
  // hold the bfloat16 pairs (x0,x2), (x4,x6), (x1,x3), (x5,x7) of the word
  // (first element in the low half); dword 16 is the fp32 sum of the unit's
  // 32 activations; 17..19 are padding.
  static constexpr int kXDw = 20;
  struct Row { const uint32_t* q; const uint16_t* s; };
  struct Raw { uint32_t q[4]; uint32_t s; };
  static __device__ __forceinline__ Row row(const uint8_t* base, const uint16_t* sc, int64_t n, int K) {
    return Row{reinterpret_cast<const uint32_t*>(base) + n * (int64_t)(K / 8), sc + n * (int64_t)(K / 32)};
  }
  static __device__ __forceinline__ int units(int K) { return K / 32; }
  static __device__ __forceinline__ int64_t row_bytes(int K) { return (int64_t)K / 2; }
  static __device__ __forceinline__ int64_t scale_row_bytes(int K) { return (int64_t)(K / 32) * 2; }
  static __device__ __forceinline__ void load(const Row& rw, int u, Raw& raw) {
    const uint4 v = *reinterpret_cast<const uint4*>(rw.q + 4 * u);
    raw.q[0] = v.x;
    raw.q[1] = v.y;
    raw.q[2] = v.z;
    raw.q[3] = v.w;
    raw.s = rw.s[u];
  }
  static __device__ __forceinline__ float dot(const Raw& raw, uint32_t, const float* __restrict__ x32) {
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
  static constexpr int kXRaw = kUnitW / 2;
  static __device__ __forceinline__ void load_x(const uint16_t* __restrict__ xt, int u, uint32_t (&p)[kXRaw]) {
#pragma unroll
    for (int c = 0; c < kXRaw / 4; ++c) load_u4(xt + kUnitW * u + 8 * c, p + 4 * c);
  }
  // Sum of the eight activations of one code word, dword by dword.
  static __device__ __forceinline__ float word_sum(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3) {
    float c = bf16_to_f32(p0 & 0xFFFFu) + bf16_to_f32(p0 >> 16);
    c += bf16_to_f32(p1 & 0xFFFFu) + bf16_to_f32(p1 >> 16);
    c += bf16_to_f32(p2 & 0xFFFFu) + bf16_to_f32(p2 >> 16);
    c += bf16_to_f32(p3 & 0xFFFFu) + bf16_to_f32(p3 >> 16);
    return c;
  }
  // The unit's sum is (c0 + c1) + (c2 + c3) over its four code words, so
  // that four threads holding eight activations each can form it.
  static __device__ __forceinline__ void pack_x(const uint32_t (&p)[kXRaw], uint32_t (&xs)[kXDw]) {
    float c[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      xs[4 * w + 0] = __builtin_amdgcn_perm(p[4 * w + 1], p[4 * w + 0], 0x05040100u);  // x0 | x2 << 16
      xs[4 * w + 1] = __builtin_amdgcn_perm(p[4 * w + 3], p[4 * w + 2], 0x05040100u);  // x4 | x6 << 16
      xs[4 * w + 2] = __builtin_amdgcn_perm(p[4 * w + 1], p[4 * w + 0], 0x07060302u);  // x1 | x3 << 16
      xs[4 * w + 3] = __builtin_amdgcn_perm(p[4 * w + 3], p[4 * w + 2], 0x07060302u);  // x5 | x7 << 16
      c[w] = word_sum(p[4 * w], p[4 * w + 1], p[4 * w + 2], p[4 * w + 3]);
    }
    xs[16] = __float_as_uint((c[0] + c[1]) + (c[2] + c[3]));
    xs[17] = xs[18] = xs[19] = 0u;
  }
  // The same staging from thread i's activations 8i..8i+7 (v): code word
  // i%4 of unit i/4.  The four threads of a unit are one lane quad; their
  // word sums meet through two DPP swaps (x + y and y + x round alike).
  // Gives the same bits as pack_x.
  static __device__ __forceinline__ void stage8(const uint4& v, int i, uint4* xt, int UG) {
    const int u = i / 4, w = i % 4;
    xt[w * UG + u] = make_uint4(__builtin_amdgcn_perm(v.y, v.x, 0x05040100u), __builtin_amdgcn_perm(v.w, v.z, 0x05040100u),
                                __builtin_amdgcn_perm(v.y, v.x, 0x07060302u), __builtin_amdgcn_perm(v.w, v.z, 0x07060302u));
    float c = word_sum(v.x, v.y, v.z, v.w);
    c += __int_as_float(dpp_i<0xB1>(__float_as_int(c), 0));  // quad_perm [1,0,3,2]: c0 + c1, c2 + c3
    c += __int_as_float(dpp_i<0x4E>(__float_as_int(c), 0));  // quad_perm [2,3,0,1]
    if (w == 0) xt[4 * UG + u] = make_uint4(__float_as_uint(c), 0u, 0u, 0u);
  }
  static __device__ __forceinline__ float gu_dot(const Raw& raw, uint32_t, const uint32_t (&xs)[kXDw]) {
    float acc = 0.0f;  // sum of u * 2^-9 * x
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t v = raw.q[w] ^ 0x88888888u;    // u = c + 8 per nibble
      const uint32_t lo = v & 0x0F0F0F0Fu;          // bytes: u0, u2, u4, u6
      const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;   // bytes: u1, u3, u5, u7
      acc = dot2_bf16(MOE_FP8X2_BF16(lo, false), xs[4 * w + 0], acc);
      acc = dot2_bf16(MOE_FP8X2_BF16(lo, true), xs[4 * w + 1], acc);
      acc = dot2_bf16(MOE_FP8X2_BF16(hi, false), xs[4 * w + 2], acc);
      acc = dot2_bf16(MOE_FP8X2_BF16(hi, true), xs[4 * w + 3], acc);
    }
    return bf16_to_f32(raw.s) * __builtin_fmaf(acc, 512.0f, -8.0f * __uint_as_float(xs[16]));
  }
  // Down projection on integer dot products.  The unit's 32 h values are
  // given as integers N_f = rint(h_f * 2^k) (|N| <= 2^22, one k per unit) in
  // six planes of balanced base-16 digits (plane p holds digit 5 - p of each
  // N, two's complement nibbles packed like the codes: element 8w + i in
  // bits 4i..4i+3 of dword 4p + w).  v_dot8_i32_i4 multiplies eight codes by
  // eight digits at once; Horner over the planes gives the exact
  // T = sum_f c_f * N_f (|T| <= 32 * 8 * 2^22 = 2^30), and the unit's
  // contribution is s * T * 2^-k.  k == kDigitPoison marks a unit with a
  // non-finite h value (the contribution is NaN).
  static constexpr bool kDigitH = true;
  static __device__ __forceinline__ float dn_dot_digits(const Raw& raw, const uint32_t (&pl)[24], int k) {
    int t = 0;
#pragma unroll
    for (int p = 0; p < 6; ++p) {
      t = p ? t * 16 : 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) t = __builtin_amdgcn_sdot8((int)raw.q[w], (int)pl[4 * p + w], t, false);
    }
    const float r = __builtin_amdgcn_ldexpf((float)t * bf16_to_f32(raw.s), -k);
    return k == kDigitPoison ? __builtin_nanf("") : r;
  }
  // Sum of one unit's h (32 values) into h[32] (fp32 h; unused with kDigitH).
  static constexpr bool kPrepH = true;
  static __device__ __forceinline__ void prep_h(float* h) {
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float4 v = *reinterpret_cast<const float4*>(h + 4 * c);
      sum += (v.x + v.y) + (v.z + v.w);
    }
    h[32] = sum;
  }
  static __device__ __forceinline__ float dn_dot(const Raw& raw, uint32_t, const float* __restrict__ h) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t v = raw.q[w] ^ 0x88888888u;
      const uint32_t lo = v & 0x0F0F0F0Fu;
      const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;
      const float4 ha = *reinterpret_cast<const float4*>(h + 8 * w);
      const float4 hb = *reinterpret_cast<const float4*>(h + 8 * w + 4);
      const f32x2 a = MOE_FP8X2_F32(lo, false);  // elements 0, 2
      const f32x2 b = MOE_FP8X2_F32(lo, true);   // 4, 6
      const f32x2 c = MOE_FP8X2_F32(hi, false);  // 1, 3
      const f32x2 d = MOE_FP8X2_F32(hi, true);   // 5, 7
      acc = __builtin_fmaf(a.x, ha.x, acc);
      acc = __builtin_fmaf(c.x, ha.y, acc);
      acc = __builtin_fmaf(a.y, ha.z, acc);
      acc = __builtin_fmaf(c.y, ha.w, acc);
      acc = __builtin_fmaf(b.x, hb.x, acc);
      acc = __builtin_fmaf(d.x, hb.y, acc);
      acc = __builtin_fmaf(b.y, hb.z, acc);
      acc = __builtin_fmaf(d.y, hb.w, acc);
    }
    return bf16_to_f32(raw.s) * __builtin_fmaf(acc, 512.0f, -8.0f * h[32]);
  }
};

}  // namespace moe
