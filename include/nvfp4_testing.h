/*
 * nvfp4_testing.h -- test hooks of libnvfp4.so.  They run the same device
 * functions the quantization kernels use, one value per thread, so that the
 * encoders can be checked exhaustively against a CPU reference.  Not part of
 * the quantization API.  All pointers are device pointers; calls are
 * asynchronous on `stream`; status codes as in nvfp4.h.
 */
#ifndef NVFP4_TESTING_H
#define NVFP4_TESTING_H

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* codes[i] = E2M1 round-to-nearest-even code (sign << 3 | magnitude) of the
 * binary32 value whose bit pattern is first + i, for i < n (n <= 2^32). */
int nvfp4_test_e2m1_rne_range(uint32_t first, int64_t n, uint8_t* codes, hipStream_t stream);

/* codes[i] = stochastic-rounding E2M1 code of y[i] with 32-bit hash h[i], in
 * groups of eight through the quantizer's packing routine; n % 8 == 0. */
int nvfp4_test_e2m1_sr(const float* y, const uint32_t* h, int64_t n, uint8_t* codes, hipStream_t stream);

/* codes[i] = block-scale code (format fmt) of the non-negative binary32
 * value whose bit pattern is first + i (first + n <= 2^31). */
int nvfp4_test_scale_encode_range(int fmt, uint32_t first, int64_t n, uint8_t* codes,
                                  hipStream_t stream);

/* out[i] = 32-bit stochastic-rounding variate of element index idx0 + i. */
int nvfp4_test_sr_hash(uint64_t seed, uint64_t idx0, int64_t n, uint32_t* out, hipStream_t stream);

/* codes[i] = MXFP8 element byte of y[i] (already divided by the block's
 * power-of-two scale) with 32-bit hash h[i]: clamped to +-448, then E4M3
 * stochastic rounding, in groups of four through the re-quantizer's packing
 * routine (every byte position of the instruction); n % 4 == 0. */
int nvfp4_test_e4m3_sr(const float* y, const uint32_t* h, int64_t n, uint8_t* codes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_TESTING_H */
