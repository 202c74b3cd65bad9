/* Sanitizer driver for the C ABI's host side (test infrastructure only).
 *
 * Linked with the library's sources compiled host-only and the runtime
 * stand-ins of hip_runtime_stubs.c, under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py).  Every entry point
 * of include/nvfp4.h and include/nvfp4_testing.h is called with valid
 * arguments (which must return NVFP4_OK and launch), with each rule of its
 * contract broken in turn (which must return NVFP4_ERR_INVALID and launch
 * nothing), and at extreme valid sizes up to NVFP4_MAX_ELEMENTS, whose
 * launch shapes must stay plausible.  The pointers stand for device memory and are
 * never dereferenced by the host code. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "nvfp4.h"
#include "nvfp4_testing.h"

extern unsigned long stub_launches, stub_bad_launches;

static int failures = 0;
static unsigned long launches_before;

static void check(int got, int want, int launched, const char *what, int line) {
  const unsigned long n = stub_launches - launches_before;
  if (got != want || (launched >= 0 && (n > 0) != (launched > 0))) {
    fprintf(stderr, "FAIL line %d (%s): status %d, expected %d; %lu launches\n", line, what, got,
            want, n);
    ++failures;
  }
}
#define CALL(want, launched, expr)                    \
  do {                                                \
    launches_before = stub_launches;                  \
    check((expr), (want), (launched), #expr, __LINE__); \
  } while (0)
#define OK_LAUNCH(expr) CALL(NVFP4_OK, 1, expr)
#define OK_NOLAUNCH(expr) CALL(NVFP4_OK, 0, expr)
#define BAD(expr) CALL(NVFP4_ERR_INVALID, 0, expr)

/* one aligned pool stands for device memory; offsets give misaligned pointers */
static _Alignas(256) unsigned char pool[1 << 16];
#define P(T, off) ((T *)(pool + (off)))
static void *ws(void) { return pool + 4096; }

static nvfp4_quant_args qargs(int64_t rows, int64_t cols, int axes) {
  nvfp4_quant_args a;
  memset(&a, 0, sizeof a);
  a.x = P(const uint16_t, 0);
  a.rows = rows;
  a.cols = cols;
  a.amax = P(const float, 256);
  a.global_fp8_max = 0.0f;
  a.scale_fmt = NVFP4_SCALE_E4M3;
  a.select = NVFP4_SELECT_4OVER6;
  a.rounding = NVFP4_ROUND_RNE;
  a.axes = axes;
  a.seed = 1;
  a.codes = P(uint8_t, 512);
  a.scales = P(uint8_t, 1024);
  a.codes_t = P(uint8_t, 1536);
  a.scales_t = P(uint8_t, 2048);
  a.count4 = NULL;
  a.workspace = NULL;
  return a;
}

static void quantize_calls(void) {
  const int64_t shapes[][2] = {{1, 16}, {16, 16}, {48, 96}, {8192, 4096}, {16384, 8192},
                               {(int64_t)1 << 22, (int64_t)1 << 22}, {(int64_t)1 << 40, 16},
                               {16, (int64_t)1 << 40}, {3, ((int64_t)1 << 40) + 16}};
  for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
    const int64_t r = shapes[s][0], c = shapes[s][1];
    for (int fmt = 0; fmt < 2; ++fmt)
      for (int sel = 0; sel <= 4; ++sel)
        for (int rnd = 0; rnd < 2; ++rnd)
          for (int axes = 1; axes <= 3; ++axes) {
            nvfp4_quant_args a = qargs(r, c, axes);
            a.scale_fmt = fmt; a.select = sel; a.rounding = rnd;
            const int valid = !(rnd == 1 && sel != 0) && !((axes & 2) && r % 16 != 0);
            if (valid) OK_LAUNCH(nvfp4_quantize(&a, 0));
            else BAD(nvfp4_quantize(&a, 0));
            if (axes == 1) {
              if (valid) OK_LAUNCH(nvfp4_quantize_rowscaled(&a, 0));
              else BAD(nvfp4_quantize_rowscaled(&a, 0));
              a.count4 = P(unsigned long long, 2560);
              a.workspace = ws();
              if (valid) OK_LAUNCH(nvfp4_quantize(&a, 0));
            }
            if ((axes == 1 || axes == 2) && sel != 4 && !(rnd == 1 && sel != 0)) {
              nvfp4_quant_args b = qargs(r, c, axes);
              b.scale_fmt = fmt; b.select = sel; b.rounding = rnd;
              const int ok = axes == 1 ? 1 : r % 16 == 0;
              if (ok) OK_LAUNCH(nvfp4_quantize_rht(&b, 5, 0));
              else BAD(nvfp4_quantize_rht(&b, 5, 0));
            }
          }
    for (int axes = 1; axes <= 3; axes += 2) {
      nvfp4_quant_args a = qargs(r, c, axes);
      a.select = NVFP4_SELECT_6;
      if (r % 16 == 0) OK_LAUNCH(nvfp4_quantize_2d(&a, 0));
      else BAD(nvfp4_quantize_2d(&a, 0));
    }
  }
  /* empty tensors: valid, nothing launched */
  nvfp4_quant_args e = qargs(0, 16, 1);
  OK_NOLAUNCH(nvfp4_quantize(&e, 0));
  e = qargs(16, 0, 3);
  OK_NOLAUNCH(nvfp4_quantize(&e, 0));
  /* each rule broken */
  nvfp4_quant_args a;
  BAD(nvfp4_quantize(NULL, 0));
  a = qargs(16, 16, 1); a.x = NULL; BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 1); a.amax = NULL; BAD(nvfp4_quantize(&a, 0));
  a = qargs(-1, 16, 1); BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, -16, 1); BAD(nvfp4_quantize(&a, 0));
  a = qargs(INT64_MAX, 16, 1); BAD(nvfp4_quantize(&a, 0));
  a = qargs((int64_t)1 << 40, (int64_t)1 << 40, 1); BAD(nvfp4_quantize(&a, 0));
  a = qargs((int64_t)1 << 31, (int64_t)1 << 31, 1); BAD(nvfp4_quantize(&a, 0));
  a = qargs(((int64_t)1 << 40) + 1, 16, 1); BAD(nvfp4_quantize(&a, 0));
  a = qargs((int64_t)1 << 22, ((int64_t)1 << 22) + 16, 3); BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 24, 1); BAD(nvfp4_quantize(&a, 0));
  a = qargs(24, 16, 2); BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 12, 2); BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 1); a.scale_fmt = 2; BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 1); a.select = -1; BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 1); a.select = 5; BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 1); a.rounding = 2; BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 1); a.rounding = NVFP4_ROUND_SR; BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 0); BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 4); BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 1); a.global_fp8_max = -1.0f; BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 1); a.global_fp8_max = NAN; BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 1); a.global_fp8_max = INFINITY; BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 1); a.codes = NULL; BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 1); a.codes = P(uint8_t, 513); BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 1); a.scales = NULL; BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 1); a.scales = P(uint8_t, 1026); BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 2); a.codes_t = NULL; BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 2); a.scales_t = NULL; BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 2); a.codes_t = P(uint8_t, 1544); BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 1); a.x = P(const uint16_t, 8); BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 1); a.amax = P(const float, 258); BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 1); a.count4 = P(unsigned long long, 2564); a.workspace = ws(); BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 1); a.count4 = P(unsigned long long, 2560); BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 1); a.count4 = P(unsigned long long, 2560); a.workspace = pool + 4100; BAD(nvfp4_quantize(&a, 0));
  a = qargs(16, 16, 2); BAD(nvfp4_quantize_rowscaled(&a, 0));
  BAD(nvfp4_quantize_rowscaled(NULL, 0));
  a = qargs(16, 16, 1); a.select = NVFP4_SELECT_4OVER6; BAD(nvfp4_quantize_2d(&a, 0));
  a = qargs(16, 16, 1); a.select = NVFP4_SELECT_6; a.rounding = NVFP4_ROUND_SR; BAD(nvfp4_quantize_2d(&a, 0));
  a = qargs(16, 16, 2); a.select = NVFP4_SELECT_6; BAD(nvfp4_quantize_2d(&a, 0));
  a = qargs(16, 24, 1); a.select = NVFP4_SELECT_6; BAD(nvfp4_quantize_2d(&a, 0));
  a = qargs(16, 16, 3); BAD(nvfp4_quantize_rht(&a, 1, 0));
  BAD(nvfp4_quantize_rht(NULL, 1, 0));
}

static void amax_calls(void) {
  const int64_t ns[] = {1, 8, 16, 1000, (int64_t)1 << 25, (int64_t)1 << 40, NVFP4_MAX_ELEMENTS};
  for (size_t i = 0; i < sizeof ns / sizeof ns[0]; ++i) {
    OK_LAUNCH(nvfp4_tensor_amax(P(const uint16_t, 0), ns[i], P(float, 256), ws(), 0));
    OK_LAUNCH(nvfp4_tensor_amax_noalloc(P(const uint16_t, 0), ns[i], P(float, 256), 0));
  }
  OK_LAUNCH(nvfp4_tensor_amax(NULL, 0, P(float, 256), ws(), 0));
  BAD(nvfp4_tensor_amax(P(const uint16_t, 0), -1, P(float, 256), ws(), 0));
  BAD(nvfp4_tensor_amax(P(const uint16_t, 0), NVFP4_MAX_ELEMENTS + 1, P(float, 256), ws(), 0));
  BAD(nvfp4_tensor_amax(P(const uint16_t, 0), INT64_MAX, P(float, 256), ws(), 0));
  BAD(nvfp4_tensor_amax_noalloc(P(const uint16_t, 0), NVFP4_MAX_ELEMENTS + 8, P(float, 256), 0));
  BAD(nvfp4_tensor_amax(NULL, 16, P(float, 256), ws(), 0));
  BAD(nvfp4_tensor_amax(P(const uint16_t, 0), 16, NULL, ws(), 0));
  BAD(nvfp4_tensor_amax(P(const uint16_t, 0), 16, P(float, 257), ws(), 0));
  BAD(nvfp4_tensor_amax(P(const uint16_t, 2), 16, P(float, 256), ws(), 0));
  BAD(nvfp4_tensor_amax(P(const uint16_t, 0), 16, P(float, 256), NULL, 0));
  BAD(nvfp4_tensor_amax(P(const uint16_t, 0), 16, P(float, 256), pool + 4104, 0));
  BAD(nvfp4_tensor_amax_noalloc(P(const uint16_t, 0), -5, P(float, 256), 0));
  BAD(nvfp4_tensor_amax_noalloc(P(const uint16_t, 0), 16, NULL, 0));
  const int64_t rs[][2] = {{1, 16}, {8192, 4096}, {(int64_t)1 << 40, 16}, {16, (int64_t)1 << 40}};
  for (size_t i = 0; i < sizeof rs / sizeof rs[0]; ++i)
    OK_LAUNCH(nvfp4_row_amax(P(const uint16_t, 0), rs[i][0], rs[i][1], P(float, 256), 0));
  OK_NOLAUNCH(nvfp4_row_amax(NULL, 0, 16, NULL, 0));
  BAD(nvfp4_row_amax(P(const uint16_t, 0), 16, 8, P(float, 256), 0));
  BAD(nvfp4_row_amax(P(const uint16_t, 0), 16, 16, P(float, 258), 0));
  for (int axis = 1; axis <= 2; ++axis) {
    OK_LAUNCH(nvfp4_rht_amax(P(const uint16_t, 0), 8192, 4096, axis, 5, P(float, 256), ws(), 0));
    OK_LAUNCH(nvfp4_rht_amax(P(const uint16_t, 0), (int64_t)1 << 36, 256, axis, 5, P(float, 256), ws(), 0));
  }
  BAD(nvfp4_rht_amax(P(const uint16_t, 0), 16, 16, 3, 5, P(float, 256), ws(), 0));
  BAD(nvfp4_rht_amax(P(const uint16_t, 0), (int64_t)1 << 37, 256, 1, 5, P(float, 256), ws(), 0));
  BAD(nvfp4_rht_amax(P(const uint16_t, 0), 16, 8, 1, 5, P(float, 256), ws(), 0));
  BAD(nvfp4_rht_amax(P(const uint16_t, 0), 8, 16, 2, 5, P(float, 256), ws(), 0));
  BAD(nvfp4_rht_amax(P(const uint16_t, 0), 16, 16, 1, 5, P(float, 256), NULL, 0));
}

static void dequantize_calls(void) {
  const int64_t shapes[][2] = {{1, 16}, {48, 96}, {8192, 4096}, {(int64_t)1 << 22, (int64_t)1 << 22},
                               {(int64_t)1 << 40, 16}, {16, (int64_t)1 << 40}};
  for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
    const int64_t r = shapes[s][0], c = shapes[s][1];
    for (int fmt = 0; fmt < 2; ++fmt) {
      OK_LAUNCH(nvfp4_dequantize(P(const uint8_t, 512), P(const uint8_t, 1024), r, c, P(const float, 256),
                                 448.0f, fmt, P(float, 3072), NULL, NULL, NULL, NULL, NULL, 0));
      OK_LAUNCH(nvfp4_dequantize(P(const uint8_t, 512), P(const uint8_t, 1024), r, c, P(const float, 256),
                                 448.0f, fmt, P(float, 3072), P(uint16_t, 3584), P(float, 3600),
                                 P(const uint16_t, 0), P(double, 3840), ws(), 0));
      OK_LAUNCH(nvfp4_dequantize_rowscaled(P(const uint8_t, 512), P(const uint8_t, 1024), r, c,
                                           P(const float, 256), 256.0f, fmt, NULL, P(uint16_t, 3584),
                                           NULL, P(const uint16_t, 0), P(double, 3840), ws(), 0));
      OK_LAUNCH(nvfp4_dequantize_rht(P(const uint8_t, 512), P(const uint8_t, 1024), r, c,
                                     P(const float, 256), 448.0f, fmt, 5, P(float, 3072), 0));
      OK_LAUNCH(nvfp4_dequantized_amax(P(const uint8_t, 512), P(const uint8_t, 1024), r, c,
                                       P(const float, 256), NULL, 448.0f, fmt, P(float, 300), ws(), 0));
      OK_LAUNCH(nvfp4_dequantized_amax(P(const uint8_t, 512), P(const uint8_t, 1024), r, c, NULL,
                                       P(const float, 256), 448.0f, fmt, P(float, 300), ws(), 0));
      const int nv_ok = r % 16 == 0, mx_ok = r % 32 == 0;
      CALL(nv_ok ? NVFP4_OK : NVFP4_ERR_INVALID, nv_ok,
           nvfp4_requantize_t(P(const uint8_t, 512), P(const uint8_t, 1024), r, c, NULL, P(const float, 256),
                              256.0f, fmt, NVFP4_TARGET_NVFP4, P(const float, 300), 0.0f, 1 - fmt, 7,
                              P(uint8_t, 1536), P(uint8_t, 2048), 0));
      CALL(mx_ok ? NVFP4_OK : NVFP4_ERR_INVALID, mx_ok,
           nvfp4_requantize_t(P(const uint8_t, 512), P(const uint8_t, 1024), r, c, P(const float, 256), NULL,
                              256.0f, fmt, NVFP4_TARGET_MXFP8, NULL, 0.0f, 0, 7, P(uint8_t, 1536),
                              P(uint8_t, 2048), 0));
    }
  }
  const uint8_t *cd = P(const uint8_t, 512), *sc = P(const uint8_t, 1024);
  const float *am = P(const float, 256);
  OK_NOLAUNCH(nvfp4_dequantize(cd, sc, 0, 16, am, 448.0f, 0, P(float, 3072), NULL, NULL, NULL, NULL, NULL, 0));
  BAD(nvfp4_dequantize(NULL, sc, 16, 16, am, 448.0f, 0, P(float, 3072), NULL, NULL, NULL, NULL, NULL, 0));
  BAD(nvfp4_dequantize(cd, NULL, 16, 16, am, 448.0f, 0, P(float, 3072), NULL, NULL, NULL, NULL, NULL, 0));
  BAD(nvfp4_dequantize(cd, sc, 16, 16, NULL, 448.0f, 0, P(float, 3072), NULL, NULL, NULL, NULL, NULL, 0));
  BAD(nvfp4_dequantize(cd, sc, 16, 24, am, 448.0f, 0, P(float, 3072), NULL, NULL, NULL, NULL, NULL, 0));
  BAD(nvfp4_dequantize(cd, sc, 16, 16, am, 0.0f, 0, P(float, 3072), NULL, NULL, NULL, NULL, NULL, 0));
  BAD(nvfp4_dequantize(cd, sc, 16, 16, am, INFINITY, 0, P(float, 3072), NULL, NULL, NULL, NULL, NULL, 0));
  BAD(nvfp4_dequantize(cd, sc, 16, 16, am, 448.0f, 3, P(float, 3072), NULL, NULL, NULL, NULL, NULL, 0));
  BAD(nvfp4_dequantize(cd, sc, 16, 16, am, 448.0f, 0, P(float, 3076), NULL, NULL, NULL, NULL, NULL, 0));
  BAD(nvfp4_dequantize(cd, sc, 16, 16, am, 448.0f, 0, NULL, NULL, P(float, 3602), NULL, NULL, NULL, 0));
  BAD(nvfp4_dequantize(cd, sc, 16, 16, am, 448.0f, 0, NULL, NULL, NULL, P(const uint16_t, 0), NULL, NULL, 0));
  BAD(nvfp4_dequantize(cd, sc, 16, 16, am, 448.0f, 0, NULL, NULL, NULL, NULL, P(double, 3840), ws(), 0));
  BAD(nvfp4_dequantize(cd, sc, 16, 16, am, 448.0f, 0, NULL, NULL, NULL, P(const uint16_t, 0), P(double, 3840), NULL, 0));
  BAD(nvfp4_dequantize(cd, sc, 16, 16, am, 448.0f, 0, NULL, NULL, NULL, P(const uint16_t, 0), P(double, 3844), ws(), 0));
  BAD(nvfp4_dequantize(P(const uint8_t, 520), sc, 16, 16, am, 448.0f, 0, P(float, 3072), NULL, NULL, NULL, NULL, NULL, 0));
  BAD(nvfp4_dequantized_amax(cd, sc, 16, 16, am, am, 448.0f, 0, P(float, 300), ws(), 0));
  BAD(nvfp4_dequantized_amax(cd, sc, 16, 16, NULL, NULL, 448.0f, 0, P(float, 300), ws(), 0));
  BAD(nvfp4_dequantized_amax(cd, sc, 16, 16, am, NULL, 448.0f, 0, P(float, 300), NULL, 0));
  BAD(nvfp4_requantize_t(cd, sc, 16, 16, am, NULL, 448.0f, 0, 2, NULL, 0.0f, 0, 0, P(uint8_t, 1536), P(uint8_t, 2048), 0));
  BAD(nvfp4_requantize_t(cd, sc, 16, 16, am, NULL, 448.0f, 0, NVFP4_TARGET_NVFP4, NULL, 0.0f, 0, 0, P(uint8_t, 1536), P(uint8_t, 2048), 0));
  BAD(nvfp4_requantize_t(cd, sc, 16, 16, am, NULL, 448.0f, 0, NVFP4_TARGET_MXFP8, NULL, 0.0f, 0, 0, P(uint8_t, 1536), P(uint8_t, 2048), 0));
  BAD(nvfp4_requantize_t(cd, sc, 32, 16, am, NULL, 448.0f, 0, NVFP4_TARGET_MXFP8, NULL, 0.0f, 0, 0, P(uint8_t, 1544), P(uint8_t, 2048), 0));
}

static void fakequant_calls(void) {
  const int64_t shapes[][2] = {{1, 16}, {14336, 4096}, {(int64_t)1 << 40, 16}};
  const uint16_t *x = P(const uint16_t, 0);
  const float *g = P(const float, 3072), *sp = P(const float, 256), *sq = P(const float, 300);
  for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
    const int64_t r = shapes[s][0], c = shapes[s][1];
    OK_LAUNCH(nvfp4_fakequant_fwd(x, r, c, sp, NULL, P(float, 5120), 0));
    OK_LAUNCH(nvfp4_fakequant_fwd(x, r, c, sp, sq, P(float, 5120), 0));
    OK_LAUNCH(nvfp4_fakequant_fwd_amax(x, r, c, sp, sq, P(float, 5120), 0));
    OK_LAUNCH(nvfp4_fakequant_bwd(x, g, r, c, sp, NULL, P(float, 5120), P(float, 6144), NULL, 0));
    OK_LAUNCH(nvfp4_fakequant_bwd(x, g, r, c, sp, sq, P(float, 5120), P(float, 6144), P(float, 6400), 0));
    OK_LAUNCH(nvfp4_fakequant_bwd_amax(x, g, r, c, sp, sq, P(float, 5120), P(float, 6144), P(float, 6400), 0));
  }
  BAD(nvfp4_fakequant_fwd(NULL, 16, 16, sp, NULL, P(float, 5120), 0));
  BAD(nvfp4_fakequant_fwd(x, 16, 16, NULL, NULL, P(float, 5120), 0));
  BAD(nvfp4_fakequant_fwd(x, 16, 24, sp, NULL, P(float, 5120), 0));
  BAD(nvfp4_fakequant_fwd(x, 16, 16, sp, NULL, NULL, 0));
  BAD(nvfp4_fakequant_fwd(x, 16, 16, P(const float, 258), NULL, P(float, 5120), 0));
  BAD(nvfp4_fakequant_bwd(x, g, 16, 16, sp, sq, P(float, 5120), P(float, 6144), NULL, 0));
  BAD(nvfp4_fakequant_bwd(x, g, 16, 16, sp, NULL, P(float, 5120), P(float, 6144), P(float, 6400), 0));
  BAD(nvfp4_fakequant_bwd(x, NULL, 16, 16, sp, NULL, P(float, 5120), P(float, 6144), NULL, 0));
  BAD(nvfp4_fakequant_bwd(x, g, -16, 16, sp, NULL, P(float, 5120), P(float, 6144), NULL, 0));
  BAD(nvfp4_fakequant_fwd(x, ((int64_t)1 << 40) + 1, 16, sp, NULL, P(float, 5120), 0));
}

static void testing_calls(void) {
  OK_LAUNCH(nvfp4_test_e2m1_rne_range(0, 1 << 20, P(uint8_t, 512), 0));
  OK_LAUNCH(nvfp4_test_e2m1_sr(P(const float, 3072), P(const uint32_t, 256), 64, P(uint8_t, 512), 0));
  OK_LAUNCH(nvfp4_test_e4m3_sr(P(const float, 3072), P(const uint32_t, 256), 64, P(uint8_t, 512), 0));
  OK_LAUNCH(nvfp4_test_sr_hash(1, (uint64_t)1 << 40, 1000, P(uint32_t, 512), 0));
  for (int fmt = 0; fmt < 2; ++fmt) OK_LAUNCH(nvfp4_test_scale_encode_range(fmt, 0, 1 << 20, P(uint8_t, 512), 0));
  BAD(nvfp4_test_e2m1_sr(P(const float, 3072), P(const uint32_t, 256), 12, P(uint8_t, 512), 0));
  BAD(nvfp4_test_e4m3_sr(P(const float, 3072), P(const uint32_t, 256), 6, P(uint8_t, 512), 0));
  BAD(nvfp4_test_sr_hash(1, 0, 10, NULL, 0));
  BAD(nvfp4_test_scale_encode_range(7, 0, 16, P(uint8_t, 512), 0));
}

int main(void) {
  if (nvfp4_abi_version() != NVFP4_ABI_VERSION || nvfp4_workspace_bytes() != NVFP4_WORKSPACE_BYTES) {
    fprintf(stderr, "ABI version or workspace size mismatch\n");
    return 1;
  }
  for (int s = -1; s <= 4; ++s)
    if (!nvfp4_status_string(s)) ++failures;
  quantize_calls();
  amax_calls();
  dequantize_calls();
  fakequant_calls();
  testing_calls();
  if (stub_bad_launches) {
    fprintf(stderr, "%lu launches with an implausible shape\n", stub_bad_launches);
    ++failures;
  }
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("abi driver: %lu launches, every status as expected\n", stub_launches);
  return 0;
}
