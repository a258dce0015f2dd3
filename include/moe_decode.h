/*
 * moe_decode.h -- C ABI of libmoedecode.so: the routed-expert matvec of
 * DeepSeek-V4-Flash-style MoE decode on AMD Instinct MI355X (gfx950).
 *
 * Every entry point takes plain pointers and sizes.  Unless stated otherwise:
 *
 *  - Pointers are DEVICE addresses of caller-owned memory (any allocator:
 *    hipMalloc, a torch tensor's data_ptr, ...).  The library never
 *    allocates, frees or retains them.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    All work is enqueued on it; results are valid once the stream has
 *    reached that point.  No entry point synchronises the host.
 *  - The return value is a moe_status.  Argument errors are detected on the
 *    host before anything is enqueued (MOE_ERR_ARG / _SHAPE / _WORKSPACE /
 *    _ALIGN); MOE_ERR_ARCH if the current device is not gfx950; MOE_ERR_HIP
 *    if a launch is rejected (moe_last_hip_error() then gives the code).
 *    Nothing is thrown across the ABI.
 *  - Calls on different streams must not share output or workspace buffers.
 *
 * Weight formats (byte layouts as the pages define them):
 *  MXFP4   17-byte blocks of 32 weights: byte 0 = E8M0 exponent e (scale
 *          2^(e-127)), bytes 1..16 = 32 E2M1 codes, element 2j in the high
 *          nibble of byte 1+j and element 2j+1 in the low nibble.
 *          [ds4.c study notes, glossary "quantization", section "MXFP4";
 *          nibble order as dequant_fp4 in the DeepSeek-V4-Flash-0731-W4A16
 *          model card's conversion script.]
 *  Q2_K    84-byte blocks of 256 weights: scales[16] at 0 (low nibble scale,
 *          high nibble min, one byte per 16 weights), qs[64] at 16 (2-bit
 *          codes, weight i in bits 2(i%4) of byte i/4), binary16 d at 80 and
 *          dmin at 82; w = d*sc*q - dmin*m.  [ds4.c study notes, glossary
 *          "quantization", section "core principle".]
 *  INT4G32 codes int32 [N][K/8], weight 8j+i of a row in bits 4i..4i+3 of
 *          word j, two's complement -8..7; scales bfloat16 [N][K/32];
 *          w = q * scale.  [DeepSeek-V4-Flash-0731-W4A16 model card,
 *          "quantization scheme": INT4, group 32, symmetric, BF16 scale.]
 *  A matrix W[N][K] is N rows of K weights, row-major, rows contiguous.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 7

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,       /* null pointer, negative or zero size where one is required */
  MOE_ERR_SHAPE = 2,     /* K not a multiple of the block length, B or top_k out of range */
  MOE_ERR_ARCH = 3,      /* the current HIP device is not gfx950 */
  MOE_ERR_HIP = 4,       /* a HIP call or kernel launch failed */
  MOE_ERR_WORKSPACE = 5, /* workspace missing, too small or not 256-byte aligned */
  MOE_ERR_ALIGN = 6,     /* a weight pointer or stride is not suitably aligned */
  MOE_ERR_SCRATCH = 7    /* moe_layer_decode_noalloc: the call needs more than the static scratch */
};

enum moe_format { MOE_FMT_MXFP4 = 0, MOE_FMT_Q2K = 1, MOE_FMT_INT4G32 = 2 };

/* Order of the quantized blocks of a weight matrix [N][K] in memory.  The
 * blocks themselves (and INT4 words and scales) are unchanged; only their
 * order differs.
 *   MOE_LAYOUT_ROWS     row-major, as the formats are published: row n holds
 *                       its K/32 (K/256 for Q2_K) blocks in order.
 *   MOE_LAYOUT_TILE256  K is cut into K/256 column tiles of 256 weights and
 *                       the tiles are stored one after the other, each
 *                       row-major: the matrix is stored as the row-major
 *                       [(K/256) * N][256] matrix whose row c*N + n holds
 *                       columns 256c .. 256c+255 of row n.  A decode kernel
 *                       that splits K over the chip's XCDs then reads one
 *                       contiguous region per XCD.  K % 256 == 0.
 *   MOE_LAYOUT_MFMA16   MXFP4 only: the TILE256 order refined for the
 *                       16x16x128 matrix-core operation.  Inside each tile
 *                       the rows are taken 16 at a time, and the 16 x 8
 *                       blocks of such a group are stored as 2 halves (tile
 *                       columns 0..127, 128..255) x 4 quarters (32 columns
 *                       each) x 16 rows: block j of row n, j = 8c + 4h + q,
 *                       is block number
 *                         (((c * N/16 + n/16) * 2 + h) * 4 + q) * 16 + n%16
 *                       of the matrix.  One 64-lane load of 17-byte blocks
 *                       then fetches a whole 16-row x 128-column operand from
 *                       contiguous memory.  N % 16 == 0, K % 256 == 0. */
enum moe_layout { MOE_LAYOUT_ROWS = 0, MOE_LAYOUT_TILE256 = 1, MOE_LAYOUT_MFMA16 = 2 };

#define MOE_MAX_TOKENS 8   /* B: one token plus up to 7 speculative drafts */
#define MOE_MAX_TOPK 8
#define MOE_MAX_EXPERTS 256

int moe_abi_version(void);
const char* moe_status_string(int status);
/* The hipError_t of the last MOE_ERR_HIP returned on this thread. */
int moe_last_hip_error(void);
/* MOE_OK if the current device is gfx950, else MOE_ERR_ARCH (or _HIP). */
int moe_device_check(void);

/* ------------------------------------------------------------------ matvec
 * y[b][n] = sum_k W[n][k] * x[b][k] for b < B, with the weights decoded
 * inside the kernel and fp32 accumulation.  x fp32 [B][K], y fp32 [B][N]
 * (overwritten).  1 <= B <= MOE_MAX_TOKENS.  W is read from memory once per
 * call for rows of up to 8192 weights (16384 for Q2_K), held in registers
 * across the B tokens; longer rows are streamed once per four tokens, the
 * later passes served by the caches.  A token's y does not depend on B (bit
 * for bit).
 * Alignment: MXFP4 and Q2_K blocks 4-byte aligned, INT4 codes 16-byte
 * aligned, x 16-byte aligned.
 * Source: the per-block decode of the formats above; the matvec against the
 * activation is the scalar reference dot of the ds4 notes ("MXFP4"), and
 * decode is bound by streaming these weights ("Mixed-precision compression
 * of DeepSeek-V4-Flash", "What compression does not solve").
 */
int moe_expert_gemv_mxfp4(const uint8_t* blocks /* [N][K/32][17] */, int N, int K,
                          const float* x, int B, float* y, void* stream);
int moe_expert_gemv_q2k(const uint8_t* blocks /* [N][K/256][84] */, int N, int K,
                        const float* x, int B, float* y, void* stream);
int moe_expert_gemv_int4g32(const int32_t* q /* [N][K/8] */, const uint16_t* scale_bf16 /* [N][K/32] */,
                            int N, int K, const float* x, int B, float* y, void* stream);

/* ------------------------------------------------------------------ alternative numerics
 * Two other ways to form the MXFP4 matvec, kept to compare numerics and
 * VALU cost with the matvec above ("ds4.c study notes", glossary page
 * "quantization").
 *
 * "MXFP4's ROCm native kernel" quantizes the activations to Q8_K and dots
 * the weights' codes with them as integers.  The pages name Q8_K without
 * defining it; here, per 256 consecutive activations of a token,
 * d = fp32(max|x| / 127) and q = clamp(rint(x / d), -127, 127) computed in
 * fp32 (IEEE division, ties to even; a block of zeros gives d = 0, q = 0).
 *   moe_q8k_quantize: x fp32 [B][K] (finite, 4-byte aligned), K % 256 == 0,
 *   B >= 1 -> q int8 [B][K], d fp32 [B][K/256] (4-byte aligned).
 *   moe_expert_gemv_mxfp4_q8: y[b][n] = sum over blocks j of
 *   2^(e_nj - 127) * d[b][j/8] * sum_i E2M1(c_nji) * q[b][32j+i]; the inner
 *   sums are exact integers (v_dot4 on doubled codes), scaled and summed in
 *   fp32.  blocks as for moe_expert_gemv_mxfp4, q 16-byte aligned,
 *   1 <= B <= MOE_MAX_TOKENS, K % 256 == 0.
 *
 * "Metal's MXFP4 -> half lookup table" decodes every weight with one
 * indexed load from a 256 x 16 table: entry [e][c] is the binary16 pattern
 * of E2M1(c) * 2^(e - 127) rounded once to nearest-even (row 255, an
 * infinite scale, holds the quiet NaN 0x7E00).  Products outside binary16's
 * range become infinities or round towards zero.
 *   moe_mxfp4_half_lut: writes the table (uint16 [256][16], device memory,
 *   2-byte aligned) as the kernels build it.
 *   moe_expert_gemv_mxfp4_hlut: y = W x with W decoded through the table
 *   (held in LDS), fp32 accumulation; arguments as moe_expert_gemv_mxfp4.
 * All four are asynchronous on `stream` and return MOE_ERR_ARG / _SHAPE /
 * _ALIGN / _ARCH before launching anything.
 */
int moe_q8k_quantize(const float* x, int B, int K, int8_t* q, float* d, void* stream);
int moe_expert_gemv_mxfp4_q8(const uint8_t* blocks /* [N][K/32][17] */, int N, int K, const int8_t* q,
                             const float* d, int B, float* y, void* stream);
int moe_mxfp4_half_lut(uint16_t* lut /* [256][16] */, void* stream);
int moe_expert_gemv_mxfp4_hlut(const uint8_t* blocks /* [N][K/32][17] */, int N, int K, const float* x, int B,
                               float* y, void* stream);

/* ------------------------------------------------------------------ routing
 * logits[b][e] = sum_k router_w[e][k] * x[b][k] accumulated in fp64; each
 * token keeps its top_k experts by logit (larger first, equal logits by
 * lower index) and gate weights softmax(selected logits).  The pages keep
 * the top 6 of 256 routed experts ("Mixed-precision compression of
 * DeepSeek-V4-Flash", "The recipe"); the softmax over the selected logits is
 * the reading used for the scoring function they leave open.
 *   router_w fp32 [E][D] (E <= 256), x bfloat16 bits [B][D], 1 <= B <= 8,
 *   1 <= top_k <= min(8, E).  Outputs: idx int32 [B][top_k] in rank order,
 *   gate_w fp32 [B][top_k]; logits_out fp64 [B][E] if not NULL.
 *   ws: >= moe_route_workspace_bytes(B, D, E, top_k) bytes, 256-byte
 *   aligned, prepared once with moe_workspace_init (the kernels leave it
 *   reusable).  Alignment: router_w 16 bytes, x_bf16 8 bytes.
 */
size_t moe_route_workspace_bytes(int B, int D, int E, int top_k);
int moe_route_topk(const float* router_w, int E, int D, const uint16_t* x_bf16, int B, int top_k,
                   int32_t* idx, float* gate_w, double* logits_out, void* ws, size_t ws_bytes,
                   void* stream);

/* ------------------------------------------------------------------ one MoE layer
 * For each token b: route (as moe_route_topk), then for every selected
 * expert e in rank order j: g = Wg_e x, u = Wu_e x, h = SiLU(g) * u (fp32,
 * SiLU(z) = z / (1 + e^-z)), yp_j = Wd_e h, and y[b] = sum_j gate_w[b][j] *
 * yp_j summed in rank order.  Tokens that pick the same expert share one read
 * of its weights ("commit more than one token per sweep of the target
 * weights": "Mixed-precision compression of DeepSeek-V4-Flash", "What
 * compression does not solve"; the width-(1+K) verify forward, "Width
 * drift").  gate/up/down are the routed experts' w1/w3/w2 projections named
 * in the W4A16 model card's quantization scheme.
 */
typedef struct moe_layer_desc {
  int format;        /* enum moe_format of gate and up (and of down unless down_format says otherwise) */
  int n_experts;     /* E <= 256 */
  int d_model;       /* D: multiple of 256 for Q2_K, of 32 otherwise */
  int d_ff;          /* F: same constraint */
  int top_k;         /* <= 8 */
  const float* router_w; /* fp32 [E][D] */
  /* Expert e's projection starts at base + e * stride (bytes).  gate and up
   * are [F][D], down is [D][F], each in `format`.  For INT4G32 these are the
   * int32 code arrays and *_scale the bfloat16 scale arrays. */
  const void* gate;
  const void* up;
  const void* down;
  int64_t gate_stride, up_stride, down_stride;
  const uint16_t* gate_scale;
  const uint16_t* up_scale;
  const uint16_t* down_scale;
  int64_t gate_scale_stride, up_scale_stride, down_scale_stride;
  int down_layout;   /* enum moe_layout of every expert's down projection
                      * (and of its INT4 scales); gate and up are row-major */
  /* Per-tensor-family precision ("Mixed-precision compression of
   * DeepSeek-V4-Flash", "The recipe": routed gate/up at 2 bits, down at
   * Q2_K): 0 = down in `format` like gate and up; otherwise 1 + the enum
   * moe_format of the down projection (then `format` covers gate and up,
   * down_scale is used only for an INT4G32 down, and d_ff must suit both
   * formats' block lengths).  A zeroed field keeps every projection in
   * `format`. */
  int down_format;
  /* Hash-routed layer ("cabbage v4x quant surgery": the first 3 of the 43
   * layers route by a fixed hash of the token id, through the tid2eid table,
   * instead of by the learned router).  NULL: learned routing.  Otherwise
   * int32 [vocab][top_k] device table whose row for token id t lists that
   * token's experts in rank order; the gate weights are the softmax over the
   * router logits of those experts (the reading used here: the pages keep a
   * gate matrix for these layers but do not give their weighting), and such a
   * layer is called through the *_ids entry points with the tokens' ids.  A
   * row that is out of range, holds an expert outside [0, n_experts) or
   * repeats one, or an id outside [0, vocab), routes that token to experts
   * 0..top_k-1 instead and sets the workspace's bad-input flag
   * (moe_workspace_flags). */
  const int32_t* tid2eid;
  int vocab;
} moe_layer_desc;
enum moe_down_format { MOE_DOWN_SAME = 0, MOE_DOWN_MXFP4 = 1, MOE_DOWN_Q2K = 2, MOE_DOWN_INT4G32 = 3 };

/* Workspace for moe_layer_decode with up to B tokens (256-byte aligned). */
size_t moe_layer_workspace_bytes(int B, int D, int F, int E, int top_k);
/* Prepare a fresh workspace (zeroes its counters); enqueued on `stream`. */
int moe_workspace_init(void* ws, size_t ws_bytes, void* stream);
/* x bfloat16 bits [B][D] (16-byte aligned); y fp32 [B][D] (overwritten,
 * 16-byte aligned).  idx_out int32 [B][top_k] and gw_out fp32 [B][top_k]
 * receive the routing if not NULL. */
int moe_layer_decode(const moe_layer_desc* L, const uint16_t* x_bf16, int B, float* y, void* ws,
                     size_t ws_bytes, int32_t* idx_out, float* gw_out, void* stream);
/* The same layer with the tokens' ids (device int32 [B]), required by a
 * hash-routed layer (tid2eid set) and ignored otherwise (may be NULL then).
 * moe_layer_decode on a hash-routed layer returns MOE_ERR_ARG. */
int moe_layer_decode_ids(const moe_layer_desc* L, const int32_t* token_ids, const uint16_t* x_bf16, int B,
                         float* y, void* ws, size_t ws_bytes, int32_t* idx_out, float* gw_out, void* stream);
/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer as moe_layer_decode, with the workspace taken from a static device
 * array inside the library instead of a caller buffer.  The array holds
 * MOE_STATIC_SCRATCH_BYTES per GPU (one copy on every device the library runs
 * on, kept until the process ends), enough for every B <= 8 at the full layer
 * shape (D 4096, F 2048, E 256, top_k 6); a call whose
 * moe_layer_workspace_bytes(B, D, F, E, top_k) exceeds it returns
 * MOE_ERR_SCRATCH before anything is enqueued.  It allocates and frees
 * nothing.  The first call on a device looks the array up,
 * clears it with a fill kernel on `stream` and synchronises `stream` once (do
 * not make that first call under graph capture); later calls enqueue the
 * layer only.  Every call on a GPU shares that GPU's array and leaves its
 * contents for the next call, so calls that overlap on one GPU (different
 * streams, or concurrent host threads) race and must be ordered by the
 * caller.  Hash-routed layers are not supported (MOE_ERR_ARG). */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)8 << 20)
int moe_layer_decode_noalloc(const moe_layer_desc* L, const uint16_t* x_bf16, int B, float* y, int32_t* idx_out,
                             float* gw_out, void* stream);
/* Sticky error flags of a layer or stack workspace, copied to the host
 * (synchronises `stream`): bit 0 a bounded wait gave up, bit 1 a hash-routed
 * layer met an invalid token id or table row.  They stay set until
 * moe_workspace_init. */
int moe_workspace_flags(const void* ws, size_t ws_bytes, uint32_t* flags, void* stream);
/* Same, recording two hipEvent_t (passed as void*) on `stream` right before
 * and right after the layer's kernels, for timing.  Either may be NULL. */
int moe_layer_decode_profiled(const moe_layer_desc* L, const uint16_t* x_bf16, int B, float* y,
                              void* ws, size_t ws_bytes, int32_t* idx_out, float* gw_out,
                              void* const* events, void* stream);

/* Diagnostic: the same layer decode with per-phase wall-clock stamps.  With
 * trace == NULL only *trace_blocks is set: the number of workgroups of the
 * single-launch kernel (0 if the shape runs as separate launches, which are
 * not traced).  Otherwise trace (device, uint64 [*trace_blocks][MOE_TRACE_FIELDS], zeroed by
 * the caller) receives, per workgroup, in slots 0..10 the 100 MHz wall clock
 * at: start, own router logits published, activations staged, all logits
 * gathered (wave 0), top-k done, grouping done, gate/up done, h slice
 * gathered, down done, partial outputs published, end; slot 11 the clock
 * when the h gather starts and slot 12 when its reads are complete; slot 13
 * the re-read passes thread 0 needed in the logit wait (bits 0..15) and in
 * the h waits (bits 16..31); slot 14 is the workgroup's XCD and slot 15 how
 * it found its index inside the XCD: bit 63 set and the index in the low
 * bits when it came from the block index (the placement probe saw workgroup
 * b on XCD b % XCDs), else the raw value of the XCD's arrival counter
 * (MOE_XCD_INDEX_ATOMIC set in the environment forces the counter). */
#define MOE_TRACE_FIELDS 16 /* uint64 per workgroup in moe_layer_decode_traced */
int moe_layer_decode_traced(const moe_layer_desc* L, const uint16_t* x_bf16, int B, float* y, void* ws,
                            size_t ws_bytes, uint64_t* trace, int* trace_blocks, void* stream);

/* ------------------------------------------------------------------ layer stack
 * Residual stream through n_layers MoE layers: for l = 0..n_layers-1,
 *   x_l = bf16_rne(h_l / sqrt(mean(h_l^2) + eps)),   h_{l+1} = h_l + moe_l(x_l),
 * with h_0 = h_in (fp32 [B][D]); the result goes to h_out (fp32 [B][D],
 * may alias h_in).  Attention is outside this path.  The norm is an
 * unweighted RMSNorm: the pages keep norms in F32 ("The recipe") without
 * defining them.  eps: 1e-6 in the stacked-layer workload.  The sum of
 * squares is taken in one fixed order (8-element chunks over 512 threads,
 * fp64), so x_l is the same whether the norm runs as its own kernel or, for
 * one token with MXFP4 MOE_LAYOUT_MFMA16 layers, inside the layer kernel.
 * ws: >= moe_stack_workspace_bytes(B, D, F, E, top_k): one layer's
 * workspace, x_l (bf16) and one fp32 residual state. */
size_t moe_stack_workspace_bytes(int B, int D, int F, int E, int top_k);
int moe_stack_decode(const moe_layer_desc* layers, int n_layers, const float* h_in, int B,
                     float* h_out, double eps, void* ws, size_t ws_bytes, void* stream);
/* The stack with the tokens' ids (device int32 [B]) for its hash-routed
 * layers; moe_stack_decode returns MOE_ERR_ARG if any layer is hash-routed. */
int moe_stack_decode_ids(const moe_layer_desc* layers, int n_layers, const int32_t* token_ids,
                         const float* h_in, int B, float* h_out, double eps, void* ws, size_t ws_bytes,
                         void* stream);
/* The norm step alone: x_out bfloat16 bits [B][D] from h fp32 [B][D]. */
int moe_rmsnorm_bf16(const float* h, int B, int D, double eps, uint16_t* x_out, void* stream);

/* ------------------------------------------------------------------ measurement
 * A pure-read yardstick: the layer streams weights from HBM, so its
 * effective bandwidth is compared with what a kernel doing nothing but reads
 * achieves with the same load patterns ("Mixed-precision compression of
 * DeepSeek-V4-Flash", "Capacity": measured pure-read bandwidth as the bound).
 * moe_stream_read reads bytes [src, src + bytes) once and writes, per
 * workgroup of its MOE_STREAM_GRID-workgroup launch, the XOR of every dword
 * it loaded to sink[workgroup] (device uint32 [MOE_STREAM_GRID]); the XOR of
 * all sink words is the XOR of the loaded dwords, which a test can check.
 *   MOE_STREAM_DWORDX4: 16-byte chunks, consecutive lanes consecutive chunks
 *     (src 16-byte aligned, bytes % 16 == 0; every dword is loaded once).
 *   MOE_STREAM_MXFP4: the 17-byte blocks of an MXFP4 array loaded as the
 *     matvecs do, the five dwords covering each block (src 4-byte aligned,
 *     bytes % 4 == 0, bytes >= 20); blocks b = 0 .. moe_stream_mxfp4_blocks(bytes)-1
 *     start at byte 17b, and the dwords from (17b & ~3) to (17b & ~3) + 16
 *     are loaded (overlapping windows are loaded twice).
 * Asynchronous on `stream`; MOE_ERR_ARG / _ALIGN / _SHAPE on bad arguments. */
#define MOE_STREAM_GRID 2048
enum moe_stream_pattern { MOE_STREAM_DWORDX4 = 0, MOE_STREAM_MXFP4 = 1 };
int moe_stream_read(const void* src, size_t bytes, int pattern, uint32_t* sink, void* stream);
/* Blocks the MXFP4 pattern reads in `bytes` bytes: the largest n whose last
 * five-dword window ends inside the range (0 if bytes < 20). */
static inline int64_t moe_stream_mxfp4_blocks(size_t bytes) {
  if (bytes < 20) return 0;
  int64_t n = (int64_t)(bytes / 17);
  while (n > 0 && ((17 * (n - 1)) & ~(int64_t)3) + 20 > (int64_t)bytes) --n;
  return n;
}

/* ------------------------------------------------------------------ FP4 -> INT4 g32
 * Per 32-weight group (= one MXFP4 block of a row): w_i = E2M1[c_i] *
 * 2^(e-127) in fp32; amax = max(max|w_i|, 1e-8); for r in {6/7, 0.9, 0.95,
 * 1.0, 1.05, 1.1} (fp32): s = fl32(fl32(amax*r)/7), q_i = clamp(rint(w_i/s),
 * -8, 7), error = sum_i (w_i - q_i*s)^2 in fp64, index order; the first
 * candidate with the strictly smallest error wins; scale = bf16_rne(s).
 * [DeepSeek-V4-Flash-0731-W4A16 model card, "FP4 -> INT4 conversion
 * algorithm", steps 1-2, and its conversion-script sketch.]
 *   mxfp4 [N][K/32][17] (4-byte aligned) -> q_out int32 [N][K/8] (16-byte
 *   aligned), scale_out bfloat16 bits [N][K/32].  Blocks with e >= 253 may
 *   overflow fp32 and e == 255 is +inf: reject them with moe_validate_mxfp4.
 */
int quantize_fp4_to_int4g32(const uint8_t* mxfp4, int N, int K, int32_t* q_out, uint16_t* scale_out,
                            void* stream);

/* ------------------------------------------------------------------ layout
 * Copies a weight matrix [N][K] of `format` from MOE_LAYOUT_ROWS (src) to
 * MOE_LAYOUT_TILE256 (dst): a permutation of whole blocks, done once when
 * the weights are loaded.  For INT4G32, src/dst are the int32 code arrays
 * and src_scale/dst_scale the bfloat16 scale arrays (else NULL).  K % 256 ==
 * 0; src and dst do not overlap; pointers 4-byte aligned (INT4 codes 16).
 * Returns MOE_ERR_SHAPE / _ALIGN / _ARG on bad arguments, before any work. */
int moe_tile_weights(int format, const void* src, const uint16_t* src_scale, int N, int K, void* dst,
                     uint16_t* dst_scale, void* stream);
/* Same for MXFP4 blocks [N][K/32][17] into MOE_LAYOUT_MFMA16 (dst).  N % 16
 * == 0 and K % 256 == 0 (MOE_ERR_SHAPE); src and dst do not overlap. */
int moe_tile_weights_mfma16(const uint8_t* src, int N, int K, uint8_t* dst, void* stream);

/* Count MXFP4 blocks whose exponent byte is 0xFF (scale +inf: infinity times
 * a zero code is NaN, which the ds4 notes treat as an error for E8M0 scales).
 * Adds the count to *bad_count_dev (device int32, caller zeroes it). */
int moe_validate_mxfp4(const uint8_t* blocks, int64_t n_blocks, int32_t* bad_count_dev, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */
