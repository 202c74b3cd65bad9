/*
 * nvfp4_oracle.c -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.
 *
 * A plain, slow CPU statement of NVFP4 block-scaled quantization, the
 * Four-Over-Six block-scale choice, stochastic rounding, and scale-learning
 * fake quantization with its straight-through gradients.  Only the tests,
 * the smoke check and the benchmark's CPU-baseline leg may load it; the
 * HIP library never links, includes or calls anything here, and nothing
 * here is shared with it.
 *
 * Sources (web pages, cited by title and section):
 *   [SL]  "Scale Learning: Training NVFP4 Block Scales to Recover Accuracy"
 *         (NVIDIA Model Optimizer blog), section "How Scale Learning Works".
 *   [UE]  "UE5M3: 给 FP4 训练算一笔更宽容的账" (blog on the UE5M3 block-scale
 *         paper), sections 背景, 数学推导, 实现.
 *   [E2E] "End-to-End 4-Bit Training" (Thinking Machines), sections
 *         "Low-precision formats on Blackwell", "Block-scaled backward
 *         passes", "Re-quantization with stochastic rounding".
 *   [46a] "Four Over Six: More Accurate NVFP4 Quantization with Adaptive
 *         Block Scaling" (gist.science summary), sections Probleemstelling,
 *         Methodologie, Implementatiedetails.
 *   [46b] same title (bud-325 notes), sections "TL;DR", "Method", "Results".
 *
 * Precision.  Where a floating-point value decides a code (a scale byte, a
 * 4-bit element code, the 4-vs-6 choice, the in-range test of the clamp) the
 * oracle takes that decision in binary32 with the operation order written
 * below, which is the order the GPU kernels use; the pages fix only that the
 * outer scale is FP32 ([E2E] Low-precision formats).  Every floating-point
 * OUTPUT (dequantized values, fake-quantized values, gradients, squared
 * error) is computed in binary64 from those decisions and rounded once to
 * binary32 at the end.  Build: gcc -O2 -ffp-contract=off, no fast-math, so
 * every float operation rounds once and fmaf() is the only fused operation.
 *
 * UE5M3 ([UE] 数学推导, 实现): unsigned, 5 exponent and 3 mantissa bits, and
 * the emulation's bias 2^(5-1) - 1 = 15 with its top binade 2^16; the tests
 * pin these against a minifloat built from those rules (the same
 * construction reproduces torch's E4M3FN byte) and against the emulation's
 * round-half-even mantissa rule over the normal range.  Still a reading:
 * the subnormals below 2^-14, 0xFF = NaN and the 114688 maximum, which carry
 * the E4M3FN conventions over (the emulation is not a format at its ends).
 */
#include <float.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_FMT_E4M3 0
#define OR_FMT_UE5M3 1
#define OR_SELECT_6 0
#define OR_SELECT_4OVER6 1        /* Four-Over-Six, smaller squared error */
#define OR_SELECT_4OVER6_MAE 2    /* Four-Over-Six, smaller absolute error */
#define OR_SELECT_4OVER6_MAXERR 3 /* Four-Over-Six, smaller largest error */
#define OR_SELECT_SWEEP 4         /* smallest squared error over every scale code */
#define OR_ROUND_RNE 0
#define OR_ROUND_SR 1

#define OR_OK 0
#define OR_EINVAL 1

/* ------------------------------------------------------------------ */
/* E2M1 element format: magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} indexed by the
 * 3-bit code, sign in bit 3 ([E2E] Low-precision formats; [UE] 背景). */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double or_e2m1_value(int code) {
  double v = E2M1_MAG[code & 7];
  return (code & 8) ? -v : v;
}

/* Nearest E2M1 magnitude to a >= 0; an exact midpoint goes to the even code
 * (round-to-nearest-even).  Anything above 6 is nearest to 6, which is the
 * clamp at q_max of [SL] How Scale Learning Works. */
static int e2m1_nearest_mag(double a) {
  if (a >= 6.0) return 7; /* nearest is 6; said outright so that huge a,
                             whose distances all round alike, cannot tie */
  int best = 0;
  double best_d = a;
  for (int k = 1; k < 8; ++k) {
    double d = fabs(a - E2M1_MAG[k]);
    if (d < best_d || (d == best_d && (k & 1) == 0)) {
      best = k;
      best_d = d;
    }
  }
  return best;
}

/* Round y to E2M1 (round-to-nearest-even), keeping the sign bit of y. */
int or_e2m1_code(float y) {
  int sign = signbit(y) ? 8 : 0;
  return sign | e2m1_nearest_mag(fabs((double)y));
}

/* Stochastic rounding of y onto E2M1 ([E2E] Re-quantization with stochastic
 * rounding; [UE] 实现): |y| goes to the grid point above it with probability
 * (|y| - lo) / (hi - lo) and to the one below otherwise.  Read as dithered
 * truncation: the fraction p = (|y| - lo) / (hi - lo), truncated to 22 bits
 * (F = floor(p * 2^22)), is added to the 22-bit variate u = h >> 10 taken from
 * the top of the 32-bit hash h; a carry out of 22 bits rounds up:
 *   up iff u + F >= 2^22,
 * so P(up) = F / 2^22, which is p exactly when p has at most 22 fractional
 * bits (every |y| >= 1) and below p by less than 2^-22 otherwise.  |y| >= 6
 * saturates to 6; the sign is kept. */
int or_e2m1_code_sr(float y, uint32_t h) {
  int sign = signbit(y) ? 8 : 0;
  double a = fabs((double)y);
  if (a >= 6.0) return sign | 7;
  int lo = 0;
  while (lo < 6 && E2M1_MAG[lo + 1] <= a) ++lo;
  double step = E2M1_MAG[lo + 1] - E2M1_MAG[lo];
  uint32_t F = (uint32_t)floor((a - E2M1_MAG[lo]) / step * 4194304.0); /* exact */
  uint32_t u = h >> 10;
  return sign | ((u + F >= (1u << 22)) ? lo + 1 : lo);
}

/* ------------------------------------------------------------------ */
/* Block-scale formats.  E4M3 is the OCP E4M3FN byte: bias 7, subnormals
 * m/8 * 2^-6, largest finite 0x7E = 448, 0x7F = NaN; this gives NVFP4 its
 * magnitude range 2^-10 .. 2688 = 6 * 448 ([E2E] Low-precision formats).
 * UE5M3 is unsigned with 5 exponent and 3 mantissa bits ([UE] 数学推导) and
 * bias 15 ([UE] 实现, the emulation's 2^(E-1) - 1); its subnormals, NaN code
 * and largest code are the reading stated in the header. */
static int fmt_max_code(int fmt) { return fmt == OR_FMT_E4M3 ? 0x7E : 0xFE; }
int or_scale_nan_code(int fmt) { return fmt == OR_FMT_E4M3 ? 0x7F : 0xFF; }

double or_scale_decode(int fmt, int code) {
  code &= 0xFF;
  if (fmt == OR_FMT_E4M3) {
    double sign = (code & 0x80) ? -1.0 : 1.0;
    int c = code & 0x7F;
    if (c == 0x7F) return NAN;
    int e = c >> 3, m = c & 7;
    return sign * (e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10));
  }
  if (code == 0xFF) return NAN;
  int e = code >> 3, m = code & 7;
  return e == 0 ? ldexp((double)m, -17) : ldexp((double)(8 + m), e - 18);
}

/* Table of the non-negative finite code values of a format. */
static void scale_table(int fmt, double *dec) {
  for (int c = 0; c <= fmt_max_code(fmt); ++c) dec[c] = or_scale_decode(fmt, c);
}

/* Encode s >= 0 to the nearest finite non-negative code value; an exact
 * midpoint goes to the even code; values above the largest finite code are
 * nearest to it (saturation).  Brute force over every code. */
static int scale_encode_tab(const double *dec, int maxc, float s) {
  double v = (double)s;
  if (v >= dec[maxc]) return maxc; /* saturation, said outright */
  int best = 0;
  double best_d = fabs(v - dec[0]);
  for (int c = 1; c <= maxc; ++c) {
    double d = fabs(v - dec[c]);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = c;
      best_d = d;
    }
  }
  return best;
}

int or_scale_encode(int fmt, float s) {
  double dec[256];
  scale_table(fmt, dec);
  return scale_encode_tab(dec, fmt_max_code(fmt), s);
}

/* ------------------------------------------------------------------ */
/* Counter-based hash for stochastic rounding.  fmix32 is the 32-bit
 * finalizer of MurmurHash3 (A. Appleby, public domain).  The variate for
 * element index idx under a 64-bit seed is fmix32(lo32(idx) ^ k) with the
 * key k = fmix32(lo32(seed) ^ fmix32(hi32(seed) ^ hi32(idx) ^ 0x9E3779B9)). */
uint32_t or_fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}

uint32_t or_sr_hash(uint64_t seed, uint64_t idx) {
  uint32_t k = or_fmix32((uint32_t)seed ^
                         or_fmix32((uint32_t)(seed >> 32) ^ (uint32_t)(idx >> 32) ^ 0x9E3779B9u));
  return or_fmix32((uint32_t)idx ^ k);
}

/* ------------------------------------------------------------------ */
/* Tensor amax: A = max |x| over the tensor ([UE] 数学推导, current-tensor
 * scaling).  Any NaN makes A NaN; otherwise an infinity makes it +inf. */
float or_tensor_amax(const float *x, int64_t n) {
  float m = 0.0f;
  int nan = 0;
  for (int64_t i = 0; i < n; ++i) {
    if (isnan(x[i])) nan = 1;
    else if (fabsf(x[i]) > m) m = fabsf(x[i]);
  }
  return nan ? NAN : m;
}

/* FP32 outer scale alpha = A / (6 * S_g): with it the largest block of the
 * tensor gets block scale S_g, the chosen FP8 maximum (448 for E4M3, 256
 * under Four-Over-Six so that a max-to-4 scale, 1.5x larger, still fits:
 * [46a] Implementatiedetails).  A = 0 gives alpha = 1.  A negative or
 * non-finite A has no scale: NaN. */
float or_alpha(float amax, float sg) {
  if (!(amax >= 0.0f) || isinf(amax)) return NAN;
  if (amax == 0.0f) return 1.0f;
  return amax / (6.0f * sg);
}

/* Per-tensor constants shared by every block (binary32, in this order):
 *   K_Q      = 1 / (Q * alpha), +inf replaced by FLT_MAX      (Q = 6 or 4)
 *   S_EFF[c] = D[c] * alpha                (effective scale of code c)
 *   INV_S[c] = 1 / S_EFF[c], or 0 if S_EFF[c] = 0 or the reciprocal is inf */
typedef struct {
  int fmt, maxc;
  double dec[256];
  float alpha, k6, k4;
  float seff[256], inv[256];
} or_consts;

static float recip_or_max(float v) {
  float r = 1.0f / v;
  return isinf(r) ? FLT_MAX : r;
}

static void make_consts(or_consts *c, int fmt, float alpha) {
  c->fmt = fmt;
  c->maxc = fmt_max_code(fmt);
  scale_table(fmt, c->dec);
  c->alpha = alpha;
  c->k6 = recip_or_max(6.0f * alpha);
  c->k4 = recip_or_max(4.0f * alpha);
  for (int k = 0; k <= c->maxc; ++k) {
    c->seff[k] = (float)c->dec[k] * alpha;
    float r = c->seff[k] == 0.0f ? 0.0f : 1.0f / c->seff[k];
    c->inv[k] = isinf(r) ? 0.0f : r;
  }
}

/* The error of one candidate encoding of a block, by the selection rule
 * ([46a] Methodologie, [46b] Key claims: the smallest maximum error, the
 * smallest absolute error (L1 / MAE), the smallest squared error (MSE); n = 16
 * is constant, so sums stand for means).  From the residuals
 * d_i = fmaf(-q_i, S_EFF, x_i):
 *   MSE:    P_k = fmaf(d_i, d_i, P_k)      over i = 4k .. 4k+3, from +0;
 *   MAE:    P_k = P_k + |d_i|              over i = 4k .. 4k+3, from +0;
 *           error = (P0 + P1) + (P2 + P3)  (binary32, this order);
 *   MAXERR: error = max |d_i|  (exact, order-free). */
static float block_error(const float d[16], int select) {
  if (select == OR_SELECT_4OVER6_MAXERR) {
    float m = 0.0f;
    for (int i = 0; i < 16; ++i)
      if (fabsf(d[i]) > m || isnan(d[i])) m = isnan(d[i]) ? NAN : fabsf(d[i]);
    return m;
  }
  float P[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int i = 0; i < 16; ++i)
    P[i / 4] = select == OR_SELECT_4OVER6_MAE ? P[i / 4] + fabsf(d[i]) : fmaf(d[i], d[i], P[i / 4]);
  return (P[0] + P[1]) + (P[2] + P[3]);
}

/* The encoding of one 16-element block under scale code `code`
 * ([E2E] Low-precision formats: value = fp4 * fp8 * fp32):
 *   y_i = x_i * INV_S[code] -> E2M1 code (RNE, or SR);
 *   d_i = fmaf(-q_i, S_EFF[code], x_i), and the block error by `select`
 *   (the squared error for max->6 and the sweep). */
static float encode_block_code(const or_consts *c, const float *xb, int code, int rounding,
                               int select, uint64_t seed, uint64_t idx0, uint8_t nib[16]) {
  float S = c->seff[code], I = c->inv[code];
  float d[16];
  for (int i = 0; i < 16; ++i) {
    float y = xb[i] * I;
    int n = rounding == OR_ROUND_SR ? or_e2m1_code_sr(y, or_sr_hash(seed, idx0 + (uint64_t)i))
                                    : or_e2m1_code(y);
    nib[i] = (uint8_t)n;
    float q = (float)or_e2m1_value(n);
    d[i] = fmaf(-q, S, xb[i]);
  }
  return block_error(d, select);
}

/* One candidate encoding with the block max mapped to Q ([UE] 数学推导:
 * s = quant(amax_b / Q_max)): s_raw = a_b * K_Q -> scale code (nearest,
 * ties to even, saturating), then encode_block_code. */
static float encode_block(const or_consts *c, const float *xb, float amax_b, float kq,
                          int rounding, int select, uint64_t seed, uint64_t idx0, int *scale_code,
                          uint8_t nib[16]) {
  float s_raw = amax_b * kq;
  int code = scale_encode_tab(c->dec, c->maxc, s_raw);
  *scale_code = code;
  return encode_block_code(c, xb, code, rounding, select, seed, idx0, nib);
}

/* Row-wise NVFP4 quantization of x[rows, cols] (cols % 16 == 0): every run of
 * 16 consecutive elements of a row is one block ([E2E] Low-precision
 * formats).  Outputs: codes[rows, cols/2] with element 2j in the low nibble
 * and 2j+1 in the high nibble of byte j; scales[rows, cols/16], one byte per
 * block.  select = Four-Over-Six encodes every block with max->6 and max->4
 * and keeps max->4 only if its SSE is strictly lower ([46b] Method; [46a]
 * Methodologie); *count4 (if given) is increased by the number of such
 * blocks.  select = 4OVER6_MAE / 4OVER6_MAXERR: the same choice by the
 * absolute-error sum or the largest error.  select = SWEEP: every finite scale
 * code is tried and the smallest squared error kept (the MSE scale sweep that
 * initializes scale learning, [SL] How Scale Learning Works and its ModelOpt
 * configuration); rounding must then be RNE and *count4 is untouched.
 * rounding = SR uses the hash of element index (row0 + r) * cols + c,
 * row0 being the global row of x's first row.  Column-wise quantization is
 * this function applied to the transpose.  sse_sel / sse6 (optional) receive
 * each block's error (by the selection rule; the squared error for max->6 and
 * the sweep) for the chosen and for the max->6 encoding.
 * A negative or non-finite amax writes the NaN scale code to every block and
 * code 0 to every element; with a usable amax, a block holding a NaN element
 * gets the NaN scale code and code 0 for its elements.  Infinite elements
 * saturate (scale at the largest code, the infinite element at +-6). */
int or_quantize(const float *x, int64_t rows, int64_t cols, int64_t row0, float amax, float sg,
                int fmt, int select, int rounding, uint64_t seed, uint8_t *codes, uint8_t *scales,
                uint64_t *count4, float *sse_sel, float *sse6) {
  if (rows < 0 || cols < 0 || cols % 16 != 0) return OR_EINVAL;
  if (fmt != OR_FMT_E4M3 && fmt != OR_FMT_UE5M3) return OR_EINVAL;
  if (select < OR_SELECT_6 || select > OR_SELECT_SWEEP) return OR_EINVAL;
  if (rounding != OR_ROUND_RNE && rounding != OR_ROUND_SR) return OR_EINVAL;
  if (rounding == OR_ROUND_SR && select != OR_SELECT_6) return OR_EINVAL;
  const int64_t nb = cols / 16;
  float alpha = or_alpha(amax, sg);
  if (isnan(alpha)) {
    memset(codes, 0, (size_t)(rows * cols / 2));
    memset(scales, or_scale_nan_code(fmt), (size_t)(rows * nb));
    for (int64_t b = 0; b < rows * nb; ++b) {
      if (sse_sel) sse_sel[b] = NAN;
      if (sse6) sse6[b] = NAN;
    }
    return OR_OK;
  }
  or_consts *c = (or_consts *)malloc(sizeof(or_consts));
  make_consts(c, fmt, alpha);
  uint64_t n4 = 0;
#pragma omp parallel for schedule(static) reduction(+ : n4)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const float *xb = x + r * cols + b * 16;
      float amax_b = 0.0f;
      int nan_b = 0;
      for (int i = 0; i < 16; ++i) {
        if (isnan(xb[i])) nan_b = 1;
        else if (fabsf(xb[i]) > amax_b) amax_b = fabsf(xb[i]);
      }
      if (nan_b) { /* a NaN element: the block has no scale */
        scales[r * nb + b] = (uint8_t)or_scale_nan_code(fmt);
        memset(codes + r * (cols / 2) + b * 8, 0, 8);
        if (sse_sel) sse_sel[r * nb + b] = NAN;
        if (sse6) sse6[r * nb + b] = NAN;
        continue;
      }
      uint64_t idx0 = (uint64_t)(row0 + r) * (uint64_t)cols + (uint64_t)(b * 16);
      uint8_t nib6[16], nib4[16], nibs[16];
      int code6, code4 = 0;
      /* the max->6 candidate's error by the block's rule (squared error for
       * max->6 itself and for the sweep) */
      const int rule = select == OR_SELECT_SWEEP ? OR_SELECT_4OVER6 : select;
      float e6 = encode_block(c, xb, amax_b, c->k6, rounding, rule, seed, idx0, &code6, nib6);
      float e = e6;
      const uint8_t *nib = nib6;
      int code = code6;
      if (select == OR_SELECT_4OVER6 || select == OR_SELECT_4OVER6_MAE ||
          select == OR_SELECT_4OVER6_MAXERR) {
        float e4 = encode_block(c, xb, amax_b, c->k4, rounding, select, seed, idx0, &code4, nib4);
        if (e4 < e6) {
          e = e4;
          nib = nib4;
          code = code4;
          n4 += 1;
        }
      } else if (select == OR_SELECT_SWEEP) {
        /* every finite scale code in ascending order; a strictly smaller
         * squared error replaces the best (ties keep the smaller code) */
        float best = INFINITY;
        for (int cc = 0; cc <= c->maxc; ++cc) {
          float ec = encode_block_code(c, xb, cc, rounding, OR_SELECT_4OVER6, seed, idx0, nibs);
          if (ec < best) {
            best = ec;
            code = cc;
            memcpy(nib4, nibs, 16);
          }
        }
        e = best;
        nib = nib4;
      }
      scales[r * nb + b] = (uint8_t)code;
      for (int j = 0; j < 8; ++j)
        codes[r * (cols / 2) + b * 8 + j] = (uint8_t)(nib[2 * j] | (nib[2 * j + 1] << 4));
      if (sse_sel) sse_sel[r * nb + b] = e;
      if (sse6) sse6[r * nb + b] = e6;
    }
  }
  free(c);
  if (count4) *count4 += n4;
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Per-row outer scales ([E2E] Recipe details: per-token outer scales when
 * quantizing activations, per-expert ones for weights).  Row r has its own
 * FP32 outer scale alpha_r = A_r / (6 * S_g), A_r = max |x| over row r (NaN
 * and infinity rules as for the tensor amax).  Everything else is the
 * per-tensor method with A replaced by A_r, so row r is quantized exactly as
 * or_quantize quantizes a one-row tensor holding that row (SR indices keep the
 * row's global position).  A per-expert outer scale is the per-tensor method
 * applied to each expert's matrix. */
int or_row_amax(const float *x, int64_t rows, int64_t cols, float *row_amax) {
  if (rows < 0 || cols < 0) return OR_EINVAL;
  for (int64_t r = 0; r < rows; ++r) row_amax[r] = or_tensor_amax(x + r * cols, cols);
  return OR_OK;
}

int or_quantize_rowscaled(const float *x, int64_t rows, int64_t cols, int64_t row0,
                          const float *row_amax, float sg, int fmt, int select, int rounding,
                          uint64_t seed, uint8_t *codes, uint8_t *scales, uint64_t *count4) {
  if (rows < 0 || cols < 0 || cols % 16 != 0) return OR_EINVAL;
  const int64_t nb = cols / 16;
  int bad = 0;
  uint64_t n4 = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(+ : n4) reduction(| : bad)
  for (int64_t r = 0; r < rows; ++r) {
    uint64_t c4 = 0;
    bad |= or_quantize(x + r * cols, 1, cols, row0 + r, row_amax[r], sg, fmt, select, rounding,
                       seed, codes + r * (cols / 2), scales + r * nb, &c4, NULL, NULL);
    n4 += c4;
  }
  if (bad) return OR_EINVAL;
  if (count4) *count4 += n4;
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* 16x16 tile scales ([E2E] Block-scaled backward passes): one block scale per
 * square 16x16 tile, from the tile's amax, shared by the tile's 16 row-wise
 * (1x16) blocks and its 16 column-wise (16x1) blocks, so that the column-wise
 * quantization is exactly the transpose of the row-wise one (w_q equals the
 * transpose of (w^T)_q, bit for bit).  Max->6, round-to-nearest-even: the
 * weights path ([E2E] Recipe details forgoes 4/6 for weights).  Requires rows
 * and cols to be multiples of 16.  Outputs the row-wise layout (codes[rows,
 * cols/2], scales[rows, cols/16]: every row block carries its tile's code)
 * and, if codes_t is given, the column-wise layout of X^T (codes_t[cols,
 * rows/2], scales_t[cols, rows/16]).  NaN rules as or_quantize, per tile. */
int or_quantize_2d(const float *x, int64_t rows, int64_t cols, float amax, float sg, int fmt,
                   uint8_t *codes, uint8_t *scales, uint8_t *codes_t, uint8_t *scales_t) {
  if (rows < 0 || cols < 0 || rows % 16 != 0 || cols % 16 != 0) return OR_EINVAL;
  if (fmt != OR_FMT_E4M3 && fmt != OR_FMT_UE5M3) return OR_EINVAL;
  const int64_t tr_n = rows / 16, tc_n = cols / 16;
  float alpha = or_alpha(amax, sg);
  or_consts *c = (or_consts *)malloc(sizeof(or_consts));
  if (!isnan(alpha)) make_consts(c, fmt, alpha);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < tr_n * tc_n; ++t) {
    const int64_t r0 = (t / tc_n) * 16, c0 = (t % tc_n) * 16;
    float at = 0.0f;
    int nan_t = isnan(alpha);
    for (int i = 0; i < 16; ++i)
      for (int j = 0; j < 16; ++j) {
        float v = x[(r0 + i) * cols + c0 + j];
        if (isnan(v)) nan_t = 1;
        else if (fabsf(v) > at) at = fabsf(v);
      }
    int code = nan_t ? or_scale_nan_code(fmt) : scale_encode_tab(c->dec, c->maxc, at * c->k6);
    float I = nan_t ? 0.0f : c->inv[code];
    for (int i = 0; i < 16; ++i) {
      scales[(r0 + i) * (cols / 16) + c0 / 16] = (uint8_t)code;
      if (scales_t) scales_t[(c0 + i) * (rows / 16) + r0 / 16] = (uint8_t)code;
      for (int j = 0; j < 16; ++j) {
        const int64_t r = r0 + i, cc = c0 + j;
        int n = nan_t ? 0 : or_e2m1_code(x[r * cols + cc] * I);
        uint8_t *b = &codes[r * (cols / 2) + cc / 2];
        *b = (uint8_t)((cc & 1) ? ((*b & 0x0F) | (n << 4)) : ((*b & 0xF0) | n));
        if (codes_t) {
          uint8_t *bt = &codes_t[cc * (rows / 2) + r / 2];
          *bt = (uint8_t)((r & 1) ? ((*bt & 0x0F) | (n << 4)) : ((*bt & 0xF0) | n));
        }
      }
    }
  }
  free(c);
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Dequantization: x_hat = q * D[scale code] * alpha ([E2E] Low-precision
 * formats: fp4 value x fp8 block scale x fp32 outer scale), the product taken
 * exactly in binary64 and rounded once to binary32; a NaN scale code gives
 * NaN.  out_bf16 (optional) is that binary32 value rounded to bfloat16 with
 * round-to-nearest-even.  block_scale (optional, [rows, cols/16]) receives
 * the binary32 effective scale D * alpha of each block. */
static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

uint16_t or_f32_to_bf16(float f) { return f32_to_bf16_rne(f); }

int or_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                  float amax, float sg, int fmt, float *out_f32, uint16_t *out_bf16,
                  float *block_scale) {
  if (rows < 0 || cols < 0 || cols % 16 != 0) return OR_EINVAL;
  if (fmt != OR_FMT_E4M3 && fmt != OR_FMT_UE5M3) return OR_EINVAL;
  const int64_t nb = cols / 16;
  const double alpha = (double)or_alpha(amax, sg);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      double D = or_scale_decode(fmt, scales[r * nb + b]);
      if (block_scale) block_scale[r * nb + b] = (float)(D * alpha);
      for (int i = 0; i < 16; ++i) {
        int64_t c = b * 16 + i;
        uint8_t byte = codes[r * (cols / 2) + c / 2];
        int nib = (c & 1) ? (byte >> 4) : (byte & 15);
        float v = (float)(or_e2m1_value(nib) * D * alpha);
        if (out_f32) out_f32[r * cols + c] = v;
        if (out_bf16) out_bf16[r * cols + c] = f32_to_bf16_rne(v);
      }
    }
  }
  return OR_OK;
}

/* Dequantization under per-row outer scales: row r uses alpha_r. */
int or_dequantize_rowscaled(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                            int64_t cols, const float *row_amax, float sg, int fmt,
                            float *out_f32, uint16_t *out_bf16, float *block_scale) {
  if (rows < 0 || cols < 0 || cols % 16 != 0) return OR_EINVAL;
  const int64_t nb = cols / 16;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
  for (int64_t r = 0; r < rows; ++r)
    bad |= or_dequantize(codes + r * (cols / 2), scales + r * nb, 1, cols, row_amax[r], sg, fmt,
                         out_f32 ? out_f32 + r * cols : NULL, out_bf16 ? out_bf16 + r * cols : NULL,
                         block_scale ? block_scale + r * nb : NULL);
  return bad ? OR_EINVAL : OR_OK;
}

/* ------------------------------------------------------------------ */
/* Re-quantization for the backward pass ([E2E] Re-quantization with
 * stochastic rounding; the quantized linear layer figure there): a tensor
 * quantized for the forward pass is dequantized, transposed in that higher
 * precision, and quantized again along the other dimension with stochastic
 * rounding, so that the backward pass sees the forward tensor in
 * expectation.  The source is the NVFP4 tensor (codes[rows, cols/2],
 * scales[rows, cols/16]) with one outer amax (row_amax == NULL) or one per
 * row; x_hat is what or_dequantize computes (q * D * alpha rounded once to
 * binary32).  Targets: NVFP4 (the max->6 quantizer of this file with SR) or
 * MXFP8 (the pages' choice for the backward GEMMs). */
static float *dequant_source(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                             int64_t cols, float amax, const float *row_amax, float sg, int fmt) {
  float *x = (float *)malloc(sizeof(float) * (size_t)(rows * cols > 0 ? rows * cols : 1));
  int bad = row_amax ? or_dequantize_rowscaled(codes, scales, rows, cols, row_amax, sg, fmt, x, NULL, NULL)
                     : or_dequantize(codes, scales, rows, cols, amax, sg, fmt, x, NULL, NULL);
  if (bad) { free(x); return NULL; }
  return x;
}

static float *transpose_f32(const float *x, int64_t rows, int64_t cols) {
  float *t = (float *)malloc(sizeof(float) * (size_t)(rows * cols > 0 ? rows * cols : 1));
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) t[c * rows + r] = x[r * cols + c];
  return t;
}

/* Amax of the dequantized tensor (current scaling of the re-quantized
 * tensor): max |x_hat|, NaN if any x_hat is NaN. */
float or_dequantized_amax(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                          float amax, const float *row_amax, float sg, int fmt) {
  float *x = dequant_source(codes, scales, rows, cols, amax, row_amax, sg, fmt);
  if (!x) return NAN;
  float m = or_tensor_amax(x, rows * cols);
  free(x);
  return m;
}

/* NVFP4 target: X_hat^T [cols, rows] quantized row-wise (blocks of 16 source
 * rows of one column) with max->6 and SR, outer amax dst_amax with S_g =
 * dst_sg; SR index = the element's index in X_hat^T ((out_row0 + c) * rows +
 * r; out_row0 > 0 when the source is a strip of columns out_row0.. of a
 * wider tensor).  rows % 16 == 0.  codes_t[cols, rows/2], scales_t[cols,
 * rows/16]. */
int or_requant_nvfp4_t(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                       float amax, const float *row_amax, float sg, int fmt, float dst_amax,
                       float dst_sg, int dst_fmt, uint64_t seed, int64_t out_row0,
                       uint8_t *codes_t, uint8_t *scales_t) {
  if (rows < 0 || cols < 0 || rows % 16 != 0 || cols % 16 != 0) return OR_EINVAL;
  float *x = dequant_source(codes, scales, rows, cols, amax, row_amax, sg, fmt);
  if (!x) return OR_EINVAL;
  float *t = transpose_f32(x, rows, cols);
  free(x);
  int st = or_quantize(t, cols, rows, out_row0, dst_amax, dst_sg, dst_fmt, OR_SELECT_6, OR_ROUND_SR,
                       seed, codes_t, scales_t, NULL, NULL, NULL);
  free(t);
  return st;
}

/* MXFP8 (OCP Microscaling; the pages name the format only): blocks of 32
 * consecutive elements share one E8M0 scale X = 2^e, elements are E4M3
 * (OCP E4M3FN, the byte of the block-scale format above) of x / X.
 *   e = floor(log2(amax_b)) - 8, clamped below at -127 (amax_b = 0 gives
 *       -127): 8 is the exponent of E4M3's largest binade, so the block's
 *       largest element lands in [256, 512);
 *   scale byte = e + 127;
 *   y_i = fl(x_i * 2^-e) (binary32), magnitudes above 448 saturate to 448;
 *   element = SR of y_i onto the E4M3 grid (or_e4m3_code_sr).
 * A block holding a NaN, or an infinity, has no representable scale: its
 * scale byte is 0xFF (E8M0's NaN) and its elements 0.
 *
 * Stochastic rounding onto E4M3 (the rule of gfx950's SR conversion to FP8,
 * of the same form as or_e2m1_code_sr with E4M3's 20 discarded mantissa
 * bits): with lo / hi the grid neighbours of a = |y| and p = (a - lo) /
 * (hi - lo), F = floor(p * 2^20) and u = h >> 12, round up iff
 * u + F >= 2^20.  a >= 448 gives 448; the sign is kept (-0 -> 0x80). */
static int e4m3_code_sr_tab(const double *dec, float y, uint32_t h) {
  int sign = signbit(y) ? 0x80 : 0;
  double a = fabs((double)y);
  if (a >= 448.0) return sign | 0x7E;
  int lo = 0;
  while (lo < 0x7E && dec[lo + 1] <= a) ++lo;
  uint32_t F = (uint32_t)floor((a - dec[lo]) / (dec[lo + 1] - dec[lo]) * 1048576.0); /* exact */
  uint32_t u = h >> 12;
  return sign | ((u + F >= (1u << 20)) ? lo + 1 : lo);
}

int or_e4m3_code_sr(float y, uint32_t h) {
  double dec[256];
  scale_table(OR_FMT_E4M3, dec);
  return e4m3_code_sr_tab(dec, y, h);
}

int or_mxfp8_quantize_sr(const float *x, int64_t rows, int64_t cols, int64_t row0, uint64_t seed,
                         uint8_t *elems, uint8_t *scales) {
  if (rows < 0 || cols < 0 || cols % 32 != 0) return OR_EINVAL;
  const int64_t nb = cols / 32;
  double dec[256];
  scale_table(OR_FMT_E4M3, dec);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const float *xb = x + r * cols + b * 32;
      uint8_t *eb = elems + r * cols + b * 32;
      float amax_b = 0.0f;
      int bad = 0;
      for (int i = 0; i < 32; ++i) {
        if (isnan(xb[i]) || isinf(xb[i])) bad = 1;
        else if (fabsf(xb[i]) > amax_b) amax_b = fabsf(xb[i]);
      }
      if (bad) {
        scales[r * nb + b] = 0xFF;
        memset(eb, 0, 32);
        continue;
      }
      int e = -127;
      if (amax_b > 0.0f) {
        int ex;
        frexpf(amax_b, &ex); /* amax_b = m * 2^ex, m in [0.5, 1): floor(log2) = ex - 1 */
        e = ex - 1 - 8;
        if (e < -127) e = -127;
      }
      scales[r * nb + b] = (uint8_t)(e + 127);
      const float inv = ldexpf(1.0f, -e);
      for (int i = 0; i < 32; ++i) {
        float y = xb[i] * inv;
        uint64_t idx = (uint64_t)(row0 + r) * (uint64_t)cols + (uint64_t)(b * 32 + i);
        eb[i] = (uint8_t)e4m3_code_sr_tab(dec, y, or_sr_hash(seed, idx));
      }
    }
  }
  return OR_OK;
}

/* MXFP8 decode: E4M3 element value * 2^(scale - 127), rounded once to
 * binary32; NaN for scale 0xFF or a NaN element. */
int or_mxfp8_dequantize(const uint8_t *elems, const uint8_t *scales, int64_t rows, int64_t cols,
                        float *out) {
  if (rows < 0 || cols < 0 || cols % 32 != 0) return OR_EINVAL;
  const int64_t nb = cols / 32;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      int sc = scales[r * nb + c / 32], el = elems[r * cols + c];
      if (sc == 0xFF || (el & 0x7F) == 0x7F) {
        out[r * cols + c] = NAN;
        continue;
      }
      double v = or_scale_decode(OR_FMT_E4M3, el & 0x7F) * ldexp(1.0, sc - 127);
      out[r * cols + c] = (float)((el & 0x80) ? -v : v);
    }
  return OR_OK;
}

/* MXFP8 target: X_hat^T [cols, rows] quantized to MXFP8 with SR along its
 * rows (blocks of 32 source rows of one column); rows % 32 == 0; SR indices
 * as for the NVFP4 target (out_row0 as there).  elems_t[cols, rows] (E4M3
 * bytes), scales_t[cols, rows/32] (E8M0). */
int or_requant_mxfp8_t(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                       float amax, const float *row_amax, float sg, int fmt, uint64_t seed,
                       int64_t out_row0, uint8_t *elems_t, uint8_t *scales_t) {
  if (rows < 0 || cols < 0 || rows % 32 != 0 || cols % 16 != 0) return OR_EINVAL;
  float *x = dequant_source(codes, scales, rows, cols, amax, row_amax, sg, fmt);
  if (!x) return OR_EINVAL;
  float *t = transpose_f32(x, rows, cols);
  free(x);
  int st = or_mxfp8_quantize_sr(t, cols, rows, out_row0, seed, elems_t, scales_t);
  free(t);
  return st;
}

/* Sum of squared errors sum (x_i - x_hat_i)^2 in binary64, in index order
 * ([UE] 实现 reports the per-tensor MSE = SSE / n). */
double or_sse(const float *x, const float *xhat, int64_t n) {
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double d = (double)x[i] - (double)xhat[i];
    s += d * d;
  }
  return s;
}

/* ------------------------------------------------------------------ */
/* Scale-learning fake quantization ([SL] How Scale Learning Works).
 *   x~ = s_post * clamp(round(x / s_pre), -6, 6),  round = nearest E2M1
 * per 16-element block with scales s_pre[b], s_post[b] (s_post == NULL:
 * tied, s_post = s_pre).  x / s_pre is taken as y = x * inv in binary32 with
 * inv = 1 / s_pre (0 if s_pre = 0; FLT_MAX-saturated if the reciprocal
 * overflows); y decides the E2M1 code and the clamp.  x~ = q * s_post
 * rounded once to binary32. */
static float fq_inv(float s) {
  if (s == 0.0f) return 0.0f;
  float r = 1.0f / s;
  return isinf(r) ? copysignf(FLT_MAX, r) : r;
}

int or_fakequant_fwd(const float *x, int64_t rows, int64_t cols, const float *s_pre,
                     const float *s_post, float *xq) {
  if (rows < 0 || cols < 0 || cols % 16 != 0) return OR_EINVAL;
  const int64_t nb = cols / 16;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      int64_t blk = r * nb + b;
      float inv = fq_inv(s_pre[blk]);
      double sp = s_post ? (double)s_post[blk] : (double)s_pre[blk];
      for (int i = 0; i < 16; ++i) {
        int64_t e = r * cols + b * 16 + i;
        float y = x[e] * inv;
        xq[e] = (float)(or_e2m1_value(or_e2m1_code(y)) * sp);
      }
    }
  }
  return OR_OK;
}

/* Straight-through backward ([SL] How Scale Learning Works), the derivative
 * of round taken as 1 and that of the FP8 scale quantization too:
 *   in_i = (-6 <= y_i <= 6)
 * Single (tied) scale:
 *   dL/dx_i = in_i ? g_i : 0
 *   dL/ds   = sum_i g_i * (in_i ? q_i - y_i : (y_i < -6 ? -6 : +6))
 * Dual scales:
 *   dL/dx_i      = in_i ? g_i * (s_post / s_pre) : 0      (0 when s_pre = 0)
 *   dL/ds_post   = sum_i g_i * clamp(q_i)                  (q_i = +-6 outside)
 *   dL/ds_pre    = sum_i g_i * (in_i ? -s_post x_i / s_pre^2 : 0)
 *                = -(s_post * T) / (s_pre * s_pre),  T = sum_{in} g_i x_i
 *                  (0 when s_pre = 0)
 * Every product and sum is binary64, summed in index order i = 0..15, and
 * rounded once to binary32.  ds_post is written only for dual scales. */
static int fq_bwd(const float *x, const float *g, int64_t rows, int64_t cols, const float *s_pre,
                  const float *s_post, double div, float *dx, float *ds_pre, float *ds_post);

int or_fakequant_bwd(const float *x, const float *g, int64_t rows, int64_t cols,
                     const float *s_pre, const float *s_post, float *dx, float *ds_pre,
                     float *ds_post) {
  return fq_bwd(x, g, rows, cols, s_pre, s_post, 1.0, dx, ds_pre, ds_post);
}

/* amax reparameterization ([SL] How Scale Learning Works: the trained
 * quantity is amax, not the scale): per block s = fl(a / 6) (binary32), the
 * fake quantization of that s, and dL/da = dL/ds * ds/da = dL/ds / 6, the
 * division applied to the binary64 block sums before their one rounding. */
static float *amax_to_scale(const float *a, int64_t n) {
  if (!a) return NULL;
  float *s = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) s[i] = a[i] / 6.0f;
  return s;
}

int or_fakequant_fwd_amax(const float *x, int64_t rows, int64_t cols, const float *a_pre,
                          const float *a_post, float *xq) {
  if (rows < 0 || cols < 0 || cols % 16 != 0) return OR_EINVAL;
  float *sp = amax_to_scale(a_pre, rows * cols / 16), *so = amax_to_scale(a_post, rows * cols / 16);
  int st = or_fakequant_fwd(x, rows, cols, sp, so, xq);
  free(sp);
  free(so);
  return st;
}

int or_fakequant_bwd_amax(const float *x, const float *g, int64_t rows, int64_t cols,
                          const float *a_pre, const float *a_post, float *dx, float *da_pre,
                          float *da_post) {
  if (rows < 0 || cols < 0 || cols % 16 != 0) return OR_EINVAL;
  float *sp = amax_to_scale(a_pre, rows * cols / 16), *so = amax_to_scale(a_post, rows * cols / 16);
  int st = fq_bwd(x, g, rows, cols, sp, so, 6.0, dx, da_pre, da_post);
  free(sp);
  free(so);
  return st;
}

/* div: the scale gradients' binary64 block sums are divided by div (1 for
 * the scale itself, 6 for the amax) before the rounding to binary32. */
static int fq_bwd(const float *x, const float *g, int64_t rows, int64_t cols, const float *s_pre,
                  const float *s_post, double div, float *dx, float *ds_pre, float *ds_post) {
  if (rows < 0 || cols < 0 || cols % 16 != 0) return OR_EINVAL;
  const int64_t nb = cols / 16;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      int64_t blk = r * nb + b;
      float sp_pre = s_pre[blk];
      float inv = fq_inv(sp_pre);
      double acc_s = 0.0, acc_post = 0.0, acc_t = 0.0;
      double ratio = 0.0;
      if (s_post && sp_pre != 0.0f) ratio = (double)s_post[blk] / (double)sp_pre;
      for (int i = 0; i < 16; ++i) {
        int64_t e = r * cols + b * 16 + i;
        float y = x[e] * inv;
        int in = (y >= -6.0f && y <= 6.0f);
        double q = or_e2m1_value(or_e2m1_code(y)); /* already clamped to +-6 */
        double gi = (double)g[e];
        if (!s_post) {
          dx[e] = in ? g[e] : 0.0f;
          double d = in ? q - (double)y : (y < -6.0f ? -6.0 : 6.0);
          acc_s += gi * d;
        } else {
          dx[e] = in ? (float)(gi * ratio) : 0.0f;
          acc_post += gi * q;
          if (in) acc_t += gi * (double)x[e];
        }
      }
      if (!s_post) {
        ds_pre[blk] = (float)(acc_s / div);
      } else {
        ds_post[blk] = (float)(acc_post / div);
        if (sp_pre == 0.0f) {
          ds_pre[blk] = 0.0f;
        } else {
          double spd = (double)sp_pre;
          ds_pre[blk] = (float)((-((double)s_post[blk] * acc_t) / (spd * spd)) / div);
        }
      }
    }
  }
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* 16-point random Hadamard transform ([46b] Method: NVIDIA's recipe applies
 * a random Hadamard transform to both inputs of the weight-gradient GEMM;
 * [E2E] Quantized communications: an orthogonal rotation that spreads
 * outliers and is inverted exactly; [UE] 背景: part of the NVFP4 recipe).
 * Per 16-element block (the NVFP4 block, along the quantized axis):
 *   y = H16 * diag(s) * x / 4,
 * H16 the Sylvester Hadamard matrix (entries +-1, H16 H16 = 16 I), s a
 * +-1 vector shared by the whole tensor: s_j = -1 iff the top bit of the
 * counter hash of (sign_seed, j) is set (j = 0..15).  Binary32, in this
 * order: t_j = x_j * (s_j * 0.25) (exact unless the result is subnormal),
 * then the fast Walsh-Hadamard butterfly, stages h = 1, 2, 4, 8, each
 * replacing (t_i, t_{i+h}) by (t_i + t_{i+h}, t_i - t_{i+h}) for the i with
 * bit h clear.  The inverse (H16 / 4 is symmetric and orthogonal):
 * t_j = y_j * 0.25, the same butterfly, then x_j = s_j * t_j. */
uint32_t or_rht_signs(uint64_t sign_seed) {
  uint32_t m = 0;
  for (int j = 0; j < 16; ++j)
    if (or_sr_hash(sign_seed, (uint64_t)j) >> 31) m |= 1u << j;
  return m;
}

static void fwht16(float t[16]) {
  for (int h = 1; h < 16; h <<= 1)
    for (int i = 0; i < 16; ++i)
      if (!(i & h)) {
        float a = t[i], b = t[i + h];
        t[i] = a + b;
        t[i + h] = a - b;
      }
}

void or_rht16(const float x[16], uint32_t signs, float y[16]) {
  for (int j = 0; j < 16; ++j) y[j] = x[j] * (((signs >> j) & 1) ? -0.25f : 0.25f);
  fwht16(y);
}

void or_irht16(const float y[16], uint32_t signs, float x[16]) {
  for (int j = 0; j < 16; ++j) x[j] = y[j] * 0.25f;
  fwht16(x);
  for (int j = 0; j < 16; ++j)
    if ((signs >> j) & 1) x[j] = -x[j];
}

/* The tensor with every block transformed: axis 1 = row blocks (16
 * consecutive elements of a row), axis 2 = column blocks (16 consecutive
 * rows of a column). */
static float *rht_tensor(const float *x, int64_t rows, int64_t cols, int axis, uint32_t signs) {
  float *y = (float *)malloc(sizeof(float) * (size_t)(rows * cols > 0 ? rows * cols : 1));
  float a[16], b[16];
  if (axis == 1) {
    for (int64_t r = 0; r < rows; ++r)
      for (int64_t c = 0; c < cols; c += 16) {
        or_rht16(x + r * cols + c, signs, b);
        memcpy(y + r * cols + c, b, sizeof b);
      }
  } else {
    for (int64_t r = 0; r < rows; r += 16)
      for (int64_t c = 0; c < cols; ++c) {
        for (int i = 0; i < 16; ++i) a[i] = x[(r + i) * cols + c];
        or_rht16(a, signs, b);
        for (int i = 0; i < 16; ++i) y[(r + i) * cols + c] = b[i];
      }
  }
  return y;
}

/* Amax of the transformed tensor (the outer scale of its quantization). */
float or_rht_amax(const float *x, int64_t rows, int64_t cols, int axis, uint64_t sign_seed) {
  if (rows < 0 || cols < 0 || (axis == 1 && cols % 16) || (axis == 2 && rows % 16) ||
      (axis != 1 && axis != 2))
    return NAN;
  float *y = rht_tensor(x, rows, cols, axis, or_rht_signs(sign_seed));
  float m = or_tensor_amax(y, rows * cols);
  free(y);
  return m;
}

/* Quantization of the transformed tensor: axis 1 = row-wise (codes[rows,
 * cols/2], scales[rows, cols/16]), axis 2 = column-wise (the layout of the
 * transposed tensor, codes[cols, rows/2], scales[cols, rows/16]); every other
 * argument as or_quantize (SR indices in the output orientation, whose first
 * row is out_row0 of a larger output when x is a strip of a larger tensor). */
int or_quantize_rht(const float *x, int64_t rows, int64_t cols, float amax, float sg, int fmt,
                    int select, int rounding, uint64_t seed, uint64_t sign_seed, int axis,
                    int64_t out_row0, uint8_t *codes, uint8_t *scales, uint64_t *count4) {
  if (rows < 0 || cols < 0 || (axis != 1 && axis != 2)) return OR_EINVAL;
  if ((axis == 1 && cols % 16) || (axis == 2 && rows % 16)) return OR_EINVAL;
  float *y = rht_tensor(x, rows, cols, axis, or_rht_signs(sign_seed));
  int st;
  if (axis == 1) {
    st = or_quantize(y, rows, cols, out_row0, amax, sg, fmt, select, rounding, seed, codes, scales,
                     count4, NULL, NULL);
  } else {
    float *t = transpose_f32(y, rows, cols);
    st = or_quantize(t, cols, rows, out_row0, amax, sg, fmt, select, rounding, seed, codes, scales,
                     count4, NULL, NULL);
    free(t);
  }
  free(y);
  return st;
}

/* Dequantization followed by the inverse transform of every row block:
 * out = RHT^-1(x_hat) (binary32), for tensors quantized row-wise by
 * or_quantize_rht with axis 1 (or column-wise, given the transposed layout). */
int or_dequantize_rht(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                      float amax, float sg, int fmt, uint64_t sign_seed, float *out) {
  int st = or_dequantize(codes, scales, rows, cols, amax, sg, fmt, out, NULL, NULL);
  if (st != OR_OK) return st;
  const uint32_t signs = or_rht_signs(sign_seed);
  float b[16];
  for (int64_t i = 0; i < rows * cols; i += 16) {
    or_irht16(out + i, signs, b);
    memcpy(out + i, b, sizeof b);
  }
  return OR_OK;
}

/* Number of OpenMP threads the parallel loops above use. */
int or_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets that number (n >= 1); the results do not depend on it. */
void or_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
