/* Sanitizer driver for the CPU oracle (test infrastructure only).
 *
 * Built together with oracle/nvfp4_oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_sanitizers.py.  Every entry point
 * runs over a grid of shapes and options on heap buffers of exactly the size
 * the function may touch, with inputs that mix normal values, zeros,
 * subnormals, infinities and NaNs, so that an access one byte out of bounds,
 * a signed overflow or a bad shift is reported.  Invalid shapes and options
 * must be rejected.  Exits non-zero on any unexpected return code. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's exported functions (oracle/nvfp4_oracle.c) */
double or_e2m1_value(int code);
int or_e2m1_code(float y);
int or_e2m1_code_sr(float y, uint32_t h);
int or_scale_nan_code(int fmt);
double or_scale_decode(int fmt, int code);
int or_scale_encode(int fmt, float s);
uint32_t or_fmix32(uint32_t h);
uint32_t or_sr_hash(uint64_t seed, uint64_t idx);
float or_tensor_amax(const float *x, int64_t n);
float or_alpha(float amax, float sg);
int or_quantize(const float *x, int64_t rows, int64_t cols, int64_t row0, float amax, float sg,
                int fmt, int select, int rounding, uint64_t seed, uint8_t *codes, uint8_t *scales,
                uint64_t *count4, float *sse_sel, float *sse6);
int or_row_amax(const float *x, int64_t rows, int64_t cols, float *row_amax);
int or_quantize_rowscaled(const float *x, int64_t rows, int64_t cols, int64_t row0,
                          const float *row_amax, float sg, int fmt, int select, int rounding,
                          uint64_t seed, uint8_t *codes, uint8_t *scales, uint64_t *count4);
int or_quantize_2d(const float *x, int64_t rows, int64_t cols, float amax, float sg, int fmt,
                   uint8_t *codes, uint8_t *scales, uint8_t *codes_t, uint8_t *scales_t);
uint16_t or_f32_to_bf16(float f);
int or_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                  float amax, float sg, int fmt, float *out_f32, uint16_t *out_bf16,
                  float *block_scale);
int or_dequantize_rowscaled(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                            int64_t cols, const float *row_amax, float sg, int fmt,
                            float *out_f32, uint16_t *out_bf16, float *block_scale);
float or_dequantized_amax(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                          float amax, const float *row_amax, float sg, int fmt);
int or_requant_nvfp4_t(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                       float amax, const float *row_amax, float sg, int fmt, float dst_amax,
                       float dst_sg, int dst_fmt, uint64_t seed, int64_t out_row0,
                       uint8_t *codes_t, uint8_t *scales_t);
int or_e4m3_code_sr(float y, uint32_t h);
int or_mxfp8_quantize_sr(const float *x, int64_t rows, int64_t cols, int64_t row0, uint64_t seed,
                         uint8_t *elems, uint8_t *scales);
int or_mxfp8_dequantize(const uint8_t *elems, const uint8_t *scales, int64_t rows, int64_t cols,
                        float *out);
int or_requant_mxfp8_t(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                       float amax, const float *row_amax, float sg, int fmt, uint64_t seed,
                       int64_t out_row0, uint8_t *elems_t, uint8_t *scales_t);
double or_sse(const float *x, const float *xhat, int64_t n);
int or_fakequant_fwd(const float *x, int64_t rows, int64_t cols, const float *s_pre,
                     const float *s_post, float *xq);
int or_fakequant_bwd(const float *x, const float *g, int64_t rows, int64_t cols,
                     const float *s_pre, const float *s_post, float *dx, float *ds_pre,
                     float *ds_post);
int or_fakequant_fwd_amax(const float *x, int64_t rows, int64_t cols, const float *a_pre,
                          const float *a_post, float *xq);
int or_fakequant_bwd_amax(const float *x, const float *g, int64_t rows, int64_t cols,
                          const float *a_pre, const float *a_post, float *dx, float *da_pre,
                          float *da_post);
uint32_t or_rht_signs(uint64_t sign_seed);
void or_rht16(const float x[16], uint32_t signs, float y[16]);
void or_irht16(const float y[16], uint32_t signs, float x[16]);
float or_rht_amax(const float *x, int64_t rows, int64_t cols, int axis, uint64_t sign_seed);
int or_quantize_rht(const float *x, int64_t rows, int64_t cols, float amax, float sg, int fmt,
                    int select, int rounding, uint64_t seed, uint64_t sign_seed, int axis,
                    int64_t out_row0, uint8_t *codes, uint8_t *scales, uint64_t *count4);
int or_dequantize_rht(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                      float amax, float sg, int fmt, uint64_t sign_seed, float *out);
int or_num_threads(void);
void or_set_num_threads(int n);

static int failures = 0;
#define EXPECT(cond, ...)                          \
  do {                                             \
    if (!(cond)) {                                 \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                \
      fprintf(stderr, "\n");                       \
      ++failures;                                  \
    }                                              \
  } while (0)

/* exact-size allocations (at least one byte, so that a zero-size buffer is
 * still a valid, unreadable-past-the-end pointer) */
static void *xmalloc(size_t n) {
  void *p = malloc(n ? n : 1);
  if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
  return p;
}

static uint64_t rng = 0x243F6A8885A308D3ull;
static uint32_t next32(void) {
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  return (uint32_t)(rng >> 16);
}

/* values of several magnitudes, with a sprinkling of specials */
static float *make_x(int64_t n, int specials) {
  float *x = (float *)xmalloc((size_t)n * sizeof(float));
  for (int64_t i = 0; i < n; ++i) {
    const uint32_t u = next32();
    float v = ((float)(u & 0xFFFF) / 65536.0f - 0.5f) * ldexpf(1.0f, (int)((u >> 16) % 24) - 12);
    if (specials) {
      switch ((u >> 24) % 64) {
        case 0: v = 0.0f; break;
        case 1: v = -0.0f; break;
        case 2: v = 1e-40f; break;        /* subnormal */
        case 3: v = 3.0e38f; break;
        case 4: if (specials > 1) v = INFINITY; break;
        case 5: if (specials > 1) v = NAN; break;
        default: break;
      }
    }
    x[i] = v;
  }
  return x;
}

static const int64_t kRows[] = {0, 1, 3, 16, 32, 48};
static const int64_t kCols[] = {16, 32, 64, 96};

static void scalars(void) {
  for (int c = 0; c < 16; ++c) (void)or_e2m1_value(c);
  for (int fmt = 0; fmt < 2; ++fmt) {
    (void)or_scale_nan_code(fmt);
    for (int code = 0; code < 256; ++code) (void)or_scale_decode(fmt, code);
  }
  const float ys[] = {0.0f, -0.0f, 0.25f, 0.75f, 1.0f, 2.5f, 5.0f, 6.0f, 7.0f, 1e30f, -1e-40f,
                      INFINITY, -INFINITY, NAN, 448.0f, 449.0f, 114688.0f, 3.4e38f};
  for (size_t i = 0; i < sizeof ys / sizeof ys[0]; ++i) {
    (void)or_e2m1_code(ys[i]);
    (void)or_f32_to_bf16(ys[i]);
    for (int fmt = 0; fmt < 2; ++fmt) (void)or_scale_encode(fmt, ys[i]);
    for (uint32_t h = 0; h < 8; ++h) {
      (void)or_e2m1_code_sr(ys[i], h * 0x2468ACE1u);
      (void)or_e4m3_code_sr(ys[i], h * 0x2468ACE1u);
    }
    for (size_t j = 0; j < sizeof ys / sizeof ys[0]; ++j) (void)or_alpha(ys[i], ys[j]);
  }
  (void)or_fmix32(0); (void)or_fmix32(0xFFFFFFFFu);
  (void)or_sr_hash(0, 0); (void)or_sr_hash(~0ull, ~0ull); (void)or_sr_hash(1ull << 40, (1ull << 33) + 5);
  float in[16], out[16], back[16];
  for (int i = 0; i < 16; ++i) in[i] = (float)(i - 7);
  const uint32_t s = or_rht_signs(12345);
  or_rht16(in, s, out);
  or_irht16(out, s, back);
  for (int i = 0; i < 16; ++i) EXPECT(fabsf(back[i] - in[i]) < 1e-5f, "rht round trip %d", i);
}

static void quantize_family(int64_t rows, int64_t cols, int specials) {
  const int64_t n = rows * cols, nb = n / 16;
  float *x = make_x(n, specials);
  const float amax = or_tensor_amax(x, n);
  uint8_t *codes = (uint8_t *)xmalloc((size_t)n / 2), *scales = (uint8_t *)xmalloc((size_t)nb);
  float *sse_sel = (float *)xmalloc((size_t)nb * 4), *sse6 = (float *)xmalloc((size_t)nb * 4);
  float *out = (float *)xmalloc((size_t)n * 4), *bsc = (float *)xmalloc((size_t)nb * 4);
  uint16_t *out16 = (uint16_t *)xmalloc((size_t)n * 2);
  float *ra = (float *)xmalloc((size_t)rows * 4);
  uint64_t count4 = 0;
  for (int fmt = 0; fmt < 2; ++fmt) {
    const float sg = fmt == 0 ? 448.0f : 114688.0f;
    for (int select = 0; select <= 4; ++select) {
      for (int rnd = 0; rnd < 2; ++rnd) {
        if (select == 4 && (rows > 16 || cols > 32)) continue; /* the sweep is slow */
        const int valid = !(rnd == 1 && select != 0);
        int rc = or_quantize(x, rows, cols, 7, amax, sg, fmt, select, rnd, 99, codes, scales, &count4,
                             sse_sel, sse6);
        EXPECT((rc == 0) == valid, "or_quantize %lldx%lld fmt %d sel %d rnd %d rc %d", (long long)rows,
               (long long)cols, fmt, select, rnd, rc);
        if (!valid) continue;
        rc = or_dequantize(codes, scales, rows, cols, amax, sg, fmt, out, out16, bsc);
        EXPECT(rc == 0, "or_dequantize rc %d", rc);
        (void)or_sse(x, out, n);
        (void)or_dequantized_amax(codes, scales, rows, cols, amax, NULL, sg, fmt);
        EXPECT(or_row_amax(x, rows, cols, ra) == 0, "or_row_amax");
        rc = or_quantize_rowscaled(x, rows, cols, 3, ra, sg, fmt, select, rnd, 5, codes, scales, &count4);
        EXPECT(rc == 0, "or_quantize_rowscaled rc %d", rc);
        rc = or_dequantize_rowscaled(codes, scales, rows, cols, ra, sg, fmt, out, out16, bsc);
        EXPECT(rc == 0, "or_dequantize_rowscaled rc %d", rc);
        (void)or_dequantized_amax(codes, scales, rows, cols, 0.0f, ra, sg, fmt);
      }
    }
    /* a NaN and a negative outer amax */
    EXPECT(or_quantize(x, rows, cols, 0, NAN, sg, fmt, 1, 0, 0, codes, scales, &count4, sse_sel, sse6) == 0,
           "nan amax");
    EXPECT(or_quantize(x, rows, cols, 0, -1.0f, sg, fmt, 0, 0, 0, codes, scales, &count4, NULL, NULL) == 0,
           "negative amax");
    EXPECT(or_dequantize(codes, scales, rows, cols, 0.0f, sg, fmt, out, NULL, NULL) == 0, "zero amax");
  }
  /* rejected options */
  EXPECT(or_quantize(x, rows, cols, 0, amax, 448.0f, 2, 0, 0, 0, codes, scales, &count4, NULL, NULL) != 0, "fmt 2");
  EXPECT(or_quantize(x, rows, cols, 0, amax, 448.0f, 0, 5, 0, 0, codes, scales, &count4, NULL, NULL) != 0, "select 5");
  EXPECT(or_quantize(x, rows, cols, 0, amax, 448.0f, 0, 0, 2, 0, codes, scales, &count4, NULL, NULL) != 0, "rnd 2");
  free(x); free(codes); free(scales); free(sse_sel); free(sse6); free(out); free(bsc); free(out16); free(ra);
}

static void transposed_family(int64_t rows, int64_t cols, int specials) {
  const int64_t n = rows * cols;
  float *x = make_x(n, specials);
  const float amax = or_tensor_amax(x, n);
  uint8_t *codes = (uint8_t *)xmalloc((size_t)n / 2), *scales = (uint8_t *)xmalloc((size_t)n / 16);
  uint8_t *codes_t = (uint8_t *)xmalloc((size_t)n / 2), *scales_t = (uint8_t *)xmalloc((size_t)n / 16);
  uint8_t *el = (uint8_t *)xmalloc((size_t)n), *msc = (uint8_t *)xmalloc((size_t)n / 32);
  float *out = (float *)xmalloc((size_t)n * 4), *ra = (float *)xmalloc((size_t)rows * 4);
  uint64_t count4 = 0;
  for (int fmt = 0; fmt < 2; ++fmt) {
    const float sg = fmt == 0 ? 448.0f : 114688.0f;
    int rc = or_quantize_2d(x, rows, cols, amax, sg, fmt, codes, scales, codes_t, scales_t);
    EXPECT(rc == 0, "or_quantize_2d rc %d", rc);
    rc = or_quantize(x, rows, cols, 0, amax, sg, fmt, 1, 0, 0, codes, scales, &count4, NULL, NULL);
    EXPECT(rc == 0, "or_quantize rc %d", rc);
    rc = or_requant_nvfp4_t(codes, scales, rows, cols, amax, NULL, sg, fmt, amax, sg, fmt, 3, 16,
                            codes_t, scales_t);
    EXPECT(rc == 0, "or_requant_nvfp4_t rc %d", rc);
    EXPECT(or_row_amax(x, rows, cols, ra) == 0, "or_row_amax");
    rc = or_requant_nvfp4_t(codes, scales, rows, cols, 0.0f, ra, sg, fmt, amax, sg, 1 - fmt, 4, 0,
                            codes_t, scales_t);
    EXPECT(rc == 0, "or_requant_nvfp4_t rowscaled rc %d", rc);
    if (rows % 32 == 0) {
      rc = or_requant_mxfp8_t(codes, scales, rows, cols, amax, NULL, sg, fmt, 9, 32, el, msc);
      EXPECT(rc == 0, "or_requant_mxfp8_t rc %d", rc);
    }
    for (int axis = 1; axis <= 2; ++axis) {
      const float ra_t = or_rht_amax(x, rows, cols, axis, 77);
      rc = or_quantize_rht(x, rows, cols, ra_t, sg, fmt, 1, 0, 0, 77, axis, 0, axis == 1 ? codes : codes_t,
                           axis == 1 ? scales : scales_t, &count4);
      EXPECT(rc == 0, "or_quantize_rht axis %d rc %d", axis, rc);
      if (axis == 1) {
        rc = or_dequantize_rht(codes, scales, rows, cols, ra_t, sg, fmt, 77, out);
        EXPECT(rc == 0, "or_dequantize_rht rc %d", rc);
      }
    }
  }
  if (cols % 32 == 0) {
    int rc = or_mxfp8_quantize_sr(x, rows, cols, 5, 11, el, msc);
    EXPECT(rc == 0, "or_mxfp8_quantize_sr rc %d", rc);
    rc = or_mxfp8_dequantize(el, msc, rows, cols, out);
    EXPECT(rc == 0, "or_mxfp8_dequantize rc %d", rc);
  }
  /* rejected shapes */
  EXPECT(or_quantize_2d(x, rows - 1, cols, amax, 448.0f, 0, codes, scales, codes_t, scales_t) != 0, "2d rows");
  EXPECT(isnan(or_rht_amax(x, rows, cols, 3, 1)), "rht axis 3");
  free(x); free(codes); free(scales); free(codes_t); free(scales_t); free(el); free(msc); free(out); free(ra);
}

static void fakequant_family(int64_t rows, int64_t cols) {
  const int64_t n = rows * cols, nb = n / 16;
  float *x = make_x(n, 1), *g = make_x(n, 1);
  float *s_pre = make_x(nb, 0), *s_post = make_x(nb, 0);
  for (int64_t b = 0; b < nb; ++b) {
    s_pre[b] = fabsf(s_pre[b]) + (b % 7 == 0 ? 0.0f : 1e-3f); /* some zero scales */
    s_post[b] = fabsf(s_post[b]) + 1e-3f;
  }
  float *xq = (float *)xmalloc((size_t)n * 4), *dx = (float *)xmalloc((size_t)n * 4);
  float *d1 = (float *)xmalloc((size_t)nb * 4), *d2 = (float *)xmalloc((size_t)nb * 4);
  EXPECT(or_fakequant_fwd(x, rows, cols, s_pre, NULL, xq) == 0, "fq fwd tied");
  EXPECT(or_fakequant_fwd(x, rows, cols, s_pre, s_post, xq) == 0, "fq fwd dual");
  EXPECT(or_fakequant_bwd(x, g, rows, cols, s_pre, NULL, dx, d1, NULL) == 0, "fq bwd tied");
  EXPECT(or_fakequant_bwd(x, g, rows, cols, s_pre, s_post, dx, d1, d2) == 0, "fq bwd dual");
  EXPECT(or_fakequant_fwd_amax(x, rows, cols, s_pre, s_post, xq) == 0, "fq fwd amax");
  EXPECT(or_fakequant_bwd_amax(x, g, rows, cols, s_pre, s_post, dx, d1, d2) == 0, "fq bwd amax");
  free(x); free(g); free(s_pre); free(s_post); free(xq); free(dx); free(d1); free(d2);
}

int main(void) {
  or_set_num_threads(2);
  (void)or_num_threads();
  scalars();
  for (size_t i = 0; i < sizeof kRows / sizeof kRows[0]; ++i)
    for (size_t j = 0; j < sizeof kCols / sizeof kCols[0]; ++j)
      for (int sp = 0; sp <= 2; ++sp) quantize_family(kRows[i], kCols[j], sp);
  for (int64_t rows = 16; rows <= 64; rows += 16)
    for (size_t j = 0; j < sizeof kCols / sizeof kCols[0]; ++j)
      for (int sp = 0; sp <= 2; ++sp) transposed_family(rows, kCols[j], sp);
  for (size_t i = 0; i < sizeof kRows / sizeof kRows[0]; ++i)
    for (size_t j = 0; j < sizeof kCols / sizeof kCols[0]; ++j) fakequant_family(kRows[i], kCols[j]);
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("oracle driver: all calls returned as expected\n");
  return 0;
}
