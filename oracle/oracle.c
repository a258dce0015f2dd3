/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU reference for the routed-expert MoE
 * decode path: block decoding of MXFP4 / Q2_K / INT4-g32 weights, matvecs,
 * router top-k with softmax, SiLU-gated expert FFN pieces, the RMSNorm used
 * between stacked layers, and the FP4 -> INT4 group-32 conversion.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load this library.  It shares no code with the GPU path.
 *
 * Arithmetic is fp64 unless the method fixes another precision (the INT4
 * conversion fixes fp32 for its scale, rounding and clamping).  Sums run in
 * ascending index order; threads split output rows only, so every output is
 * computed by one sequential loop and the result does not depend on the
 * thread count.  Build with -ffp-contract=off.
 *
 * Sources (page title, section):
 *  [ds4-q]  ds4.c study notes, glossary page "quantization": the Q2_K block
 *           under "core principle", the MXFP4 struct, code table and scalar
 *           reference under "MXFP4 -- microscaling float".
 *  [w4a16]  Model card "DeepSeek-V4-Flash-0731-W4A16": "quantization scheme"
 *           (INT4, group 32, symmetric, BF16 scale) and "FP4 -> INT4
 *           conversion algorithm", steps 1 and 2, plus the conversion-script
 *           sketch (dequant_fp4 / quant_int4).
 *  [mixed]  "Mixed-precision compression of DeepSeek-V4-Flash": "The recipe"
 *           (256 routed experts, top-6 kept), "What compression does not
 *           solve" (decode streams the active weights).
 *  [ds4-q] also: "Metal's MXFP4 -> half lookup table" (the 256 x 16 table of
 *           exactly rounded binary16 products) and "MXFP4's ROCm native
 *           kernel" (activations quantized to Q8_K, integer dot products).
 *
 * Every function below is pinned by tests/test_oracle_pins.py (the stacked
 * composition, in oracle/__init__.py, by its special cases as well).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NOMEM 2

/* ------------------------------------------------------------ scalar formats */

/* E2M1 (OCP FP4): 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit.  The
 * sixteen values this yields are the code table printed in [ds4-q] MXFP4 and
 * in [w4a16] step 1 (codes 8..15 are the negatives of codes 0..7). */
double oracle_e2m1(int code) {
  const int sign = (code >> 3) & 1;
  const int ex = (code >> 1) & 3;
  const int man = code & 1;
  double mag;
  if (ex == 0)
    mag = 0.5 * man; /* subnormal: 0 or 0.5 */
  else
    mag = ldexp(1.0 + 0.5 * man, ex - 1);
  return sign ? -mag : mag;
}

/* E8M0 shared exponent: 2^(e-127).  [ds4-q] MXFP4 reads it as the fp32 bit
 * pattern e<<23, so e == 0 is the subnormal 2^-127 (which the formula also
 * gives) and e == 255 is +infinity. */
double oracle_e8m0(int e) {
  if (e == 255) return INFINITY;
  return ldexp(1.0, e - 127);
}

double oracle_f16_to_double(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(m + 1024), e - 25);
  return s ? -v : v;
}

double oracle_bf16_to_double(uint16_t b) {
  const int s = b >> 15, e = (b >> 7) & 0xFF, m = b & 0x7F;
  double v;
  if (e == 0)
    v = ldexp((double)m, -133);
  else if (e == 255)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(m + 128), e - 134);
  return s ? -v : v;
}

/* Round a double to the nearest bfloat16, ties to even (no intermediate
 * rounding to fp32). */
uint16_t oracle_bf16_rne(double v) {
  if (isnan(v)) return 0x7FC0;
  const int neg = signbit(v) ? 1 : 0;
  double a = fabs(v);
  uint16_t bits;
  if (a == 0.0) {
    bits = 0;
  } else if (isinf(a)) {
    bits = 0x7F80;
  } else {
    int ex;
    frexp(a, &ex);           /* a = f * 2^ex, f in [0.5, 1) */
    int E = ex - 1;          /* a in [2^E, 2^(E+1)) */
    if (E < -126) E = -126;  /* subnormal range shares the quantum 2^-133 */
    const double quantum = ldexp(1.0, E - 7);
    const double n = rint(a / quantum); /* exact scaling, then ties-to-even */
    const double r = n * quantum;
    const float f = (float)r; /* exactly representable, or overflows to inf */
    uint32_t u;
    memcpy(&u, &f, 4);
    bits = (uint16_t)(u >> 16);
  }
  return (uint16_t)(bits | (neg << 15));
}

/* ------------------------------------------------------------ block decoders */

/* MXFP4 block ([ds4-q] MXFP4): byte 0 is the E8M0 exponent e, bytes 1..16
 * hold 32 four-bit codes.  Element 2j is the high nibble of code byte j and
 * element 2j+1 the low nibble (the order of dequant_fp4 in [w4a16], whose
 * packing [ds4-q] says GGUF copies byte for byte).  w = E2M1[c] * 2^(e-127),
 * exact in fp64. */
void oracle_mxfp4_decode(const uint8_t* blocks, int64_t nblocks, double* w) {
  for (int64_t b = 0; b < nblocks; ++b) {
    const uint8_t* blk = blocks + 17 * b;
    const double scale = oracle_e8m0(blk[0]);
    for (int j = 0; j < 16; ++j) {
      const uint8_t byte = blk[1 + j];
      w[32 * b + 2 * j] = oracle_e2m1(byte >> 4) * scale;
      w[32 * b + 2 * j + 1] = oracle_e2m1(byte & 0xF) * scale;
    }
  }
}

/* Q2_K block ([ds4-q] "core principle": scales[16], qs[64], f16 d, f16 dmin,
 * 84 bytes per 256 weights).  Read: scales at byte 0, qs at 16, d at 80, dmin
 * at 82 (little-endian binary16).  Sub-block j = i/16 owns scales[j], whose
 * low nibble is the scale sc and high nibble the min m.  Weight i's 2-bit
 * code is bits 2*(i%4).. of qs[i/4].  w = d*sc*q - dmin*m (the page prints a
 * garbled form; this is the asymmetric reading it describes), exact in fp64. */
void oracle_q2k_decode(const uint8_t* blocks, int64_t nblocks, double* w) {
  for (int64_t b = 0; b < nblocks; ++b) {
    const uint8_t* blk = blocks + 84 * b;
    const uint8_t* scales = blk;
    const uint8_t* qs = blk + 16;
    const double d = oracle_f16_to_double((uint16_t)(blk[80] | (blk[81] << 8)));
    const double dmin = oracle_f16_to_double((uint16_t)(blk[82] | (blk[83] << 8)));
    for (int i = 0; i < 256; ++i) {
      const int j = i / 16;
      const int sc = scales[j] & 0xF;
      const int m = scales[j] >> 4;
      const int q = (qs[i / 4] >> (2 * (i % 4))) & 3;
      w[256 * b + i] = d * sc * q - dmin * m;
    }
  }
}

/* INT4 group-32 symmetric with BF16 scale ([w4a16] scheme; packing "8 x int4
 * -> 1 x int32").  Group G covers 32 weights: code words 4G..4G+3, element
 * 8j+i of the group in bits 4i..4i+3 of word j, two's complement (-8..7).
 * w = q * scale. */
void oracle_int4g32_decode(const int32_t* q, const uint16_t* scales, int64_t ngroups, double* w) {
  for (int64_t g = 0; g < ngroups; ++g) {
    const double s = oracle_bf16_to_double(scales[g]);
    for (int i = 0; i < 32; ++i) {
      const uint32_t word = (uint32_t)q[4 * g + i / 8];
      int v = (int)((word >> (4 * (i % 8))) & 0xF);
      if (v >= 8) v -= 16;
      w[32 * g + i] = v * s;
    }
  }
}

/* ------------------------------------------------------------ threading */

typedef void (*row_fn)(void* ctx, int64_t row, double* scratch);

typedef struct {
  row_fn fn;
  void* ctx;
  int64_t begin, end;
  int64_t scratch_len;
  int status;
} row_job;

static void* row_worker(void* p) {
  row_job* job = (row_job*)p;
  double* scratch = NULL;
  if (job->scratch_len > 0) {
    scratch = (double*)malloc(sizeof(double) * (size_t)job->scratch_len);
    if (!scratch) {
      job->status = ORACLE_ERR_NOMEM;
      return NULL;
    }
  }
  for (int64_t r = job->begin; r < job->end; ++r) job->fn(job->ctx, r, scratch);
  free(scratch);
  job->status = ORACLE_OK;
  return NULL;
}

static int for_rows(row_fn fn, void* ctx, int64_t nrows, int64_t scratch_len, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > nrows) nthreads = (int)(nrows > 0 ? nrows : 1);
  row_job jobs[256];
  pthread_t tid[256];
  const int64_t per = (nrows + nthreads - 1) / nthreads;
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].fn = fn;
    jobs[t].ctx = ctx;
    jobs[t].begin = t * per < nrows ? t * per : nrows;
    jobs[t].end = (t + 1) * per < nrows ? (t + 1) * per : nrows;
    jobs[t].scratch_len = scratch_len;
    jobs[t].status = ORACLE_OK;
  }
  if (nthreads == 1) {
    row_worker(&jobs[0]);
    return jobs[0].status;
  }
  for (int t = 0; t < nthreads; ++t) {
    if (pthread_create(&tid[t], NULL, row_worker, &jobs[t]) != 0) break;
    ++started;
  }
  for (int t = started; t < nthreads; ++t) row_worker(&jobs[t]);
  for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
  for (int t = 0; t < nthreads; ++t)
    if (jobs[t].status != ORACLE_OK) return jobs[t].status;
  return ORACLE_OK;
}

/* ------------------------------------------------------------ matvec */

enum { ORACLE_FMT_MXFP4 = 0, ORACLE_FMT_Q2K = 1, ORACLE_FMT_INT4G32 = 2 };

typedef struct {
  int fmt;
  const void* w0;
  const void* w1;
  int N, K, B;
  const double* x;
  double* y;
} gemv_ctx;

static void decode_row(const gemv_ctx* c, int64_t n, double* row) {
  const int64_t K = c->K;
  if (c->fmt == ORACLE_FMT_MXFP4) {
    oracle_mxfp4_decode((const uint8_t*)c->w0 + n * (K / 32) * 17, K / 32, row);
  } else if (c->fmt == ORACLE_FMT_Q2K) {
    oracle_q2k_decode((const uint8_t*)c->w0 + n * (K / 256) * 84, K / 256, row);
  } else {
    oracle_int4g32_decode((const int32_t*)c->w0 + n * (K / 8), (const uint16_t*)c->w1 + n * (K / 32),
                          K / 32, row);
  }
}

static void gemv_row(void* p, int64_t n, double* row) {
  const gemv_ctx* c = (const gemv_ctx*)p;
  decode_row(c, n, row);
  for (int b = 0; b < c->B; ++b) {
    const double* x = c->x + (int64_t)b * c->K;
    double acc = 0.0;
    for (int k = 0; k < c->K; ++k) acc += row[k] * x[k];
    c->y[(int64_t)b * c->N + n] = acc;
  }
}

/* y[b, n] = sum_k W[n, k] * x[b, k] in fp64, k ascending.  W is N rows of K
 * weights, row-major, in format fmt (w0 = blocks or INT4 code words, w1 =
 * INT4 scales).  K must be a multiple of the format's block length. */
int oracle_gemv(int fmt, const void* w0, const void* w1, int N, int K, const double* x, int B,
                double* y, int nthreads) {
  if (!w0 || !x || !y || N < 0 || B < 0 || K <= 0) return ORACLE_ERR_ARG;
  if (fmt == ORACLE_FMT_Q2K ? (K % 256) : (K % 32)) return ORACLE_ERR_ARG;
  if (fmt == ORACLE_FMT_INT4G32 && !w1) return ORACLE_ERR_ARG;
  if (fmt < 0 || fmt > 2) return ORACLE_ERR_ARG;
  gemv_ctx c = {fmt, w0, w1, N, K, B, x, y};
  return for_rows(gemv_row, &c, N, K, nthreads);
}

/* Dequantised rows, for tests: W[n, k] as fp64, [N, K]. */
int oracle_dequant(int fmt, const void* w0, const void* w1, int N, int K, double* out) {
  if (!w0 || !out || N < 0 || K <= 0) return ORACLE_ERR_ARG;
  if (fmt == ORACLE_FMT_Q2K ? (K % 256) : (K % 32)) return ORACLE_ERR_ARG;
  gemv_ctx c = {fmt, w0, w1, N, K, 0, NULL, NULL};
  for (int64_t n = 0; n < N; ++n) decode_row(&c, n, out + n * (int64_t)K);
  return ORACLE_OK;
}

/* ------------------------------------------------------------ routing */

typedef struct {
  const float* Wr;
  int E, D, B;
  const double* x;
  double* logits;
} router_ctx;

static void router_row(void* p, int64_t e, double* unused) {
  (void)unused;
  const router_ctx* c = (const router_ctx*)p;
  const float* w = c->Wr + e * (int64_t)c->D;
  for (int b = 0; b < c->B; ++b) {
    const double* x = c->x + (int64_t)b * c->D;
    double acc = 0.0;
    for (int k = 0; k < c->D; ++k) acc += (double)w[k] * x[k];
    c->logits[(int64_t)b * c->E + e] = acc;
  }
}

/* Router logits [B, E] = x [B, D] times Wr[E, D]^T, fp64. */
int oracle_router_logits(const float* Wr, int E, int D, const double* x, int B, double* logits,
                         int nthreads) {
  if (!Wr || !x || !logits || E <= 0 || D <= 0 || B < 0) return ORACLE_ERR_ARG;
  router_ctx c = {Wr, E, D, B, x, logits};
  return for_rows(router_row, &c, E, 0, nthreads);
}

/* Top-k by logit, largest first, equal logits ordered by lower expert index;
 * then softmax over the k selected logits (fp64, max-subtracted, sum in rank
 * order).  The pages fix top-6 of 256 ([mixed] "The recipe") but not the
 * scoring function; a plain softmax over the selected logits is the reading. */
int oracle_topk_softmax(const double* logits, int E, int B, int k, int32_t* idx, double* g) {
  if (!logits || !idx || !g || k <= 0 || k > E || B < 0) return ORACLE_ERR_ARG;
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  if (!taken) return ORACLE_ERR_NOMEM;
  for (int b = 0; b < B; ++b) {
    const double* l = logits + (int64_t)b * E;
    memset(taken, 0, (size_t)E);
    for (int r = 0; r < k; ++r) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict: ties keep the lower index */
      }
      taken[best] = 1;
      idx[b * k + r] = best;
    }
    const double m = l[idx[b * k]];
    double sum = 0.0;
    for (int r = 0; r < k; ++r) {
      g[b * k + r] = exp(l[idx[b * k + r]] - m);
      sum += g[b * k + r];
    }
    for (int r = 0; r < k; ++r) g[b * k + r] /= sum;
  }
  free(taken);
  return ORACLE_OK;
}

/* Hash-routed layer ("cabbage v4x quant surgery": the first 3 of the 43
 * layers map each token to experts by a fixed hash of its id, the tid2eid
 * table, independent of the weights): token b uses experts
 * table[ids[b]][0..k-1] in that order.  Its gate weights are the softmax over
 * those experts' router logits (fp64, shifted by the largest of them, summed
 * in table order) -- a reading: the pages keep a gate matrix for these layers
 * without saying how it weighs the experts.  An id outside [0, vocab), or a
 * row with an expert outside [0, E) or a repeated one, routes the token to
 * experts 0..k-1; *n_bad counts such tokens. */
int oracle_hash_route(const double* logits, int E, int B, int k, const int32_t* table, int vocab,
                      const int32_t* ids, int32_t* idx, double* g, int* n_bad) {
  if (!logits || !table || !ids || !idx || !g || !n_bad || k <= 0 || k > E || B < 0 || vocab <= 0)
    return ORACLE_ERR_ARG;
  *n_bad = 0;
  for (int b = 0; b < B; ++b) {
    const double* l = logits + (int64_t)b * E;
    int ok = ids[b] >= 0 && ids[b] < vocab;
    const int32_t* row = table + (int64_t)(ok ? ids[b] : 0) * k;
    for (int r = 0; r < k && ok; ++r) {
      if (row[r] < 0 || row[r] >= E) ok = 0;
      for (int q = 0; q < r && ok; ++q)
        if (row[q] == row[r]) ok = 0;
    }
    if (!ok) ++*n_bad;
    for (int r = 0; r < k; ++r) idx[b * k + r] = ok ? row[r] : r;
    double m = l[idx[b * k]];
    for (int r = 1; r < k; ++r)
      if (l[idx[b * k + r]] > m) m = l[idx[b * k + r]];
    double sum = 0.0;
    for (int r = 0; r < k; ++r) {
      g[b * k + r] = exp(l[idx[b * k + r]] - m);
      sum += g[b * k + r];
    }
    for (int r = 0; r < k; ++r) g[b * k + r] /= sum;
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------ expert FFN pieces */

/* SiLU(z) = z * sigmoid(z) = z / (1 + e^-z).  Not defined on the pages; this
 * is the textbook gate of a SiLU-gated FFN. */
double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/* h[i] = silu(gate[i]) * up[i]. */
void oracle_silu_mul(const double* gate, const double* up, int64_t n, double* h) {
  for (int64_t i = 0; i < n; ++i) h[i] = oracle_silu(gate[i]) * up[i];
}

/* Between stacked layers: x = bf16_rne(h / sqrt(mean(h^2) + eps)) per token
 * row of length D (an unweighted RMSNorm; the pages keep norms in F32 but do
 * not define them, so this is a reading). */
void oracle_rmsnorm_bf16(const double* h, int B, int D, double eps, uint16_t* out) {
  for (int b = 0; b < B; ++b) {
    const double* r = h + (int64_t)b * D;
    double ss = 0.0;
    for (int i = 0; i < D; ++i) ss += r[i] * r[i];
    const double denom = sqrt(ss / D + eps);
    for (int i = 0; i < D; ++i) out[(int64_t)b * D + i] = oracle_bf16_rne(r[i] / denom);
  }
}

/* ------------------------------------------------------------ FP4 -> INT4 g32 */

/* The six round-rate candidates of [w4a16] step 2, as the fp32 values a
 * float32 tensor computation uses for those Python doubles. */
static float cand(int j) {
  switch (j) {
    case 0: return (float)(6.0 / 7.0);
    case 1: return (float)0.9;
    case 2: return (float)0.95;
    case 3: return (float)1.0;
    case 4: return (float)1.05;
    default: return (float)1.1;
  }
}

float oracle_int4_candidate(int j) { return cand(j); }

/* Convert each MXFP4 block (one 32-weight group of a row) to INT4 group-32
 * ([w4a16] "FP4 -> INT4 conversion algorithm" and the conversion sketch):
 *   1. w_i = E2M1[c_i] * 2^(e-127) as fp32 (exact for the normal range).
 *   2. amax = max(max_i |w_i|, 1e-8) in fp32.
 *   3. For each candidate r in order: s = fl32(fl32(amax*r)/7),
 *      q_i = clamp(round_half_even(fl32(w_i/s)), -8, 7), and the group's
 *      squared error sum_i (w_i - q_i*s)^2, taken here in fp64 in index order
 *      (the page averages in fp32 without fixing an order; the fp64 sum is the
 *      reading, and the 1/32 of the mean does not change the argmin).
 *      A candidate replaces the best only if its error is strictly smaller.
 *   4. scale = bf16_rne(s_best); codes packed 8 per int32 word, element i of
 *      a word in bits 4i..4i+3.
 * If s_out is not NULL, the fp32 winning s is stored per group; if r_out is
 * not NULL, the index of the winning candidate. */
int oracle_quantize_fp4_to_int4g32(const uint8_t* mx, int64_t ngroups, int32_t* q_out,
                                   uint16_t* scale_out, float* s_out, int32_t* r_out) {
  if (!mx || !q_out || !scale_out || ngroups < 0) return ORACLE_ERR_ARG;
  for (int64_t g = 0; g < ngroups; ++g) {
    const uint8_t* blk = mx + 17 * g;
    double wd[32];
    oracle_mxfp4_decode(blk, 1, wd);
    float w[32];
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
      w[i] = (float)wd[i];
      const float a = fabsf(w[i]);
      if (a > amax) amax = a;
    }
    const float floor_amax = (float)1e-8;
    if (amax < floor_amax) amax = floor_amax;
    double best_err = INFINITY;
    int best_j = -1;
    float best_s = 0.0f;
    int best_q[32];
    for (int j = 0; j < 6; ++j) {
      const float prod = amax * cand(j);
      const float s = prod / 7.0f;
      int q[32];
      double err = 0.0;
      for (int i = 0; i < 32; ++i) {
        float r = rintf(w[i] / s);
        if (r < -8.0f) r = -8.0f;
        if (r > 7.0f) r = 7.0f;
        q[i] = (int)r;
        const double diff = (double)w[i] - (double)q[i] * (double)s;
        err += diff * diff;
      }
      if (err < best_err) {
        best_err = err;
        best_j = j;
        best_s = s;
        memcpy(best_q, q, sizeof(q));
      }
    }
    for (int wi = 0; wi < 4; ++wi) {
      uint32_t word = 0;
      for (int i = 0; i < 8; ++i) word |= ((uint32_t)best_q[8 * wi + i] & 0xFu) << (4 * i);
      q_out[4 * g + wi] = (int32_t)word;
    }
    scale_out[g] = oracle_bf16_rne((double)best_s);
    if (s_out) s_out[g] = best_s;
    if (r_out) r_out[g] = best_j;
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ alternative numerics
 * [ds4-q] "MXFP4's ROCm native kernel": the activations are quantized to
 * Q8_K on the GPU and the weights' codes are dotted with them as integers.
 * The pages name Q8_K but do not define it; the reading used here: for every
 * 256 consecutive activations of a token, d = fp32(max|x| / 127) and
 * q = clamp(rint(x / d), -127, 127), both in fp32 (IEEE division, ties to
 * even); a block of zeros has d = 0 and q = 0.
 */
int oracle_q8k_quantize(const float* x, int B, int K, int8_t* q, float* d) {
  if (!x || !q || !d || B < 1 || K < 256 || K % 256) return ORACLE_ERR_ARG;
  for (int t = 0; t < B; ++t) {
    for (int b = 0; b < K / 256; ++b) {
      const float* xb = x + (int64_t)t * K + 256 * b;
      float amax = 0.0f;
      for (int i = 0; i < 256; ++i) {
        const float a = fabsf(xb[i]);
        if (a > amax) amax = a;
      }
      const float db = amax / 127.0f;
      d[(int64_t)t * (K / 256) + b] = db;
      for (int i = 0; i < 256; ++i) {
        float r = db > 0.0f ? rintf(xb[i] / db) : 0.0f;
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[(int64_t)t * K + 256 * b + i] = (int8_t)r;
      }
    }
  }
  return ORACLE_OK;
}

/* y[t][n] = sum over blocks j of 2^(e - 127) * d[t][j / 8] * sum_i E2M1(c_i) *
 * q[t][32 j + i]: the MXFP4 weights against the Q8 activations.  Twice an
 * E2M1 value is an integer (0..12), so the inner sum is an exact integer and
 * every block term is exact in fp64; terms are added in block order.
 * absy[t][n] receives the sum of the terms' magnitudes (for error bounds). */
int oracle_gemv_mxfp4_q8(const uint8_t* blocks, int N, int K, const int8_t* q, const float* d, int B, double* y,
                         double* absy) {
  if (!blocks || !q || !d || !y || N < 1 || K < 256 || K % 256 || B < 1) return ORACLE_ERR_ARG;
  for (int t = 0; t < B; ++t) {
    for (int n = 0; n < N; ++n) {
      double acc = 0.0, aacc = 0.0;
      for (int j = 0; j < K / 32; ++j) {
        const uint8_t* blk = blocks + ((int64_t)n * (K / 32) + j) * 17;
        long isum = 0;
        for (int i = 0; i < 32; ++i) {
          const int code = (i % 2 == 0) ? (blk[1 + i / 2] >> 4) : (blk[1 + i / 2] & 0xF);
          const long c2 = (long)(2.0 * oracle_e2m1(code));
          isum += c2 * (long)q[(int64_t)t * K + 32 * j + i];
        }
        const double term = (double)isum * ldexp(1.0, (int)blk[0] - 128) * (double)d[(int64_t)t * (K / 256) + j / 8];
        acc += term;
        aacc += fabs(term);
      }
      y[(int64_t)t * N + n] = acc;
      if (absy) absy[(int64_t)t * N + n] = aacc;
    }
  }
  return ORACLE_OK;
}

/* [ds4-q] "Metal's MXFP4 -> half lookup table": entry [e][c] is the binary16
 * pattern of E2M1(c) * 2^(e - 127), rounded once to nearest-even with exact
 * integer arithmetic.  The pages keep an arithmetic path for e = 255 (an
 * infinite scale); reading: that row holds the quiet NaN 0x7E00. */
static uint16_t half_of_scaled_code(int e, int code) {
  const uint16_t sign = (code & 8) ? 0x8000 : 0;
  const int m = (int)(2.0 * fabs(oracle_e2m1(code)));  /* |value| = m * 2^(e - 128), m in 0..12 */
  if (m == 0) return sign;
  const int k = e - 128;
  int L = 0;  /* bit length of m */
  while ((m >> L) != 0) ++L;
  const int E = k + L - 1;  /* |value| = 1.f * 2^E */
  if (E > 15) return sign | 0x7C00;  /* overflow: m has at most 4 significant bits, so no rounding reaches it */
  if (E >= -14) {
    /* normal: 10 fraction bits hold m's L - 1 fraction bits exactly */
    const int frac = (m << (10 - (L - 1))) & 0x3FF;
    return sign | (uint16_t)(((E + 15) << 10) | frac);
  }
  /* subnormal: count of 2^-24 units = m * 2^(k + 24), rounded to nearest-even */
  const int s = k + 24;
  if (s >= 0) return sign | (uint16_t)(m << s);
  const int sh = -s;
  if (sh > 6) return sign; /* m * 2^-sh < 12/128 < 1/2: rounds to zero */
  const int whole = m >> sh, rem = m & ((1 << sh) - 1), half = 1 << (sh - 1);
  int r = whole;
  if (rem > half || (rem == half && (whole & 1))) ++r;
  return sign | (uint16_t)r;
}

void oracle_mxfp4_half_lut(uint16_t* out) {
  for (int e = 0; e < 256; ++e)
    for (int c = 0; c < 16; ++c) out[e * 16 + c] = e == 255 ? 0x7E00 : half_of_scaled_code(e, c);
}

/* y[t][n] = sum_k half(W[n][k]) * x[t][k] in fp64, the weights decoded
 * through the table above (k ascending). */
int oracle_gemv_mxfp4_half(const uint8_t* blocks, int N, int K, const double* x, int B, double* y) {
  if (!blocks || !x || !y || N < 1 || K < 32 || K % 32 || B < 1) return ORACLE_ERR_ARG;
  uint16_t* lut = (uint16_t*)malloc(256 * 16 * sizeof(uint16_t));
  if (!lut) return ORACLE_ERR_ARG;
  oracle_mxfp4_half_lut(lut);
  for (int t = 0; t < B; ++t) {
    for (int n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int k = 0; k < K; ++k) {
        const uint8_t* blk = blocks + ((int64_t)n * (K / 32) + k / 32) * 17;
        const int i = k % 32;
        const int code = (i % 2 == 0) ? (blk[1 + i / 2] >> 4) : (blk[1 + i / 2] & 0xF);
        acc += oracle_f16_to_double(lut[blk[0] * 16 + code]) * x[(int64_t)t * K + k];
      }
      y[(int64_t)t * N + n] = acc;
    }
  }
  free(lut);
  return ORACLE_OK;
}
