/*
 * nvfp4.h -- NVFP4 block-scaled quantization of bfloat16 tensors on AMD
 * Instinct MI355X (gfx950).  C ABI of libnvfp4.so.
 *
 * The method (sources are web pages, cited by title and section):
 *  - NVFP4: every 16 consecutive values share one 8-bit block scale; each
 *    value is a 4-bit E2M1 code with magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6};
 *    a binary32 per-tensor outer scale alpha shifts the range, and a value is
 *    reconstructed as fp4 x fp8 x fp32 ("End-to-End 4-Bit Training",
 *    section "Low-precision formats on Blackwell").
 *  - Block scale = block amax / Q_max encoded to E4M3 (or to UE5M3, "UE5M3:
 *    给 FP4 训练算一笔更宽容的账", section 数学推导).
 *  - Four-Over-Six: encode each block with its max mapped to 6 and to 4 and
 *    keep the lower-squared-error result ("Four Over Six: More Accurate NVFP4
 *    Quantization with Adaptive Block Scaling", gist.science summary section
 *    Methodologie and bud-325 notes section "Method"); under it the outer
 *    scale maps the tensor amax to an FP8 maximum of 256, not 448 (gist.science
 *    summary, section Implementatiedetails).
 *  - Stochastic rounding for gradients only ("UE5M3" blog, 数学推导;
 *    "End-to-End 4-Bit Training", "Re-quantization with stochastic rounding").
 *  - Column-wise blocks for the transposed operand ("End-to-End 4-Bit
 *    Training", "Block-scaled backward passes").
 *  - Scale-learning fake quantization and its straight-through gradients,
 *    single and dual (pre/post) scales ("Scale Learning: Training NVFP4 Block
 *    Scales to Recover Accuracy", section "How Scale Learning Works").
 *
 * Conventions shared by every entry point
 *  - All data pointers are DEVICE pointers (hipMalloc'd or torch CUDA/HIP
 *    tensors) unless stated; the caller owns every buffer; the library keeps
 *    no state between calls and allocates nothing.
 *  - Every call is asynchronous on `stream` (NULL = the null stream) and
 *    never synchronizes.
 *  - Workspace: calls that combine one value per workgroup across the whole
 *    launch (a maximum, a count, a sum) take `workspace`, NVFP4_WORKSPACE_BYTES
 *    of device memory (16-byte aligned) that the caller zero-fills once before
 *    its first use.  Each workgroup stores its value in its own slot and the
 *    last one to finish combines the slots in a fixed order, in the same
 *    launch (the 4/6 count instead travels in the workgroups' arrivals at a
 *    few group counters and is added to the output per group: integer sums
 *    do not depend on the order); every call that runs to completion leaves the workspace's
 *    counters zero again, so it is reused as is.  Calls that may run at the
 *    same time (other streams) need workspaces of their own.
 *  - Arguments are validated on the host before anything is launched; a
 *    non-zero status means nothing was launched (NVFP4_ERR_HIP: a launch was
 *    attempted and HIP reported an error).
 *  - Sizes: rows, cols and numel are >= 0 and a tensor holds at most
 *    NVFP4_MAX_ELEMENTS elements; anything else -> NVFP4_ERR_INVALID.
 *  - bfloat16 values travel as their 16-bit patterns (uint16_t).
 *  - Tensors are dense row-major [rows, cols].  Data pointers (x, codes,
 *    out_f32, out_bf16, grad tensors) must be 16-byte aligned; the row-wise
 *    scale array of nvfp4_quantize 4-byte aligned; other per-block arrays
 *    need only their natural alignment.
 *  - Packed codes: byte j of a row holds element 2j in its low nibble and
 *    element 2j+1 in its high nibble; nibble = sign << 3 | magnitude index.
 *    Scales: one byte per 16-element block, [rows, cols/16], row-major.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 8

/* Size of a workspace (see the conventions above). */
#define NVFP4_WORKSPACE_BYTES 66688

/* Largest tensor any call accepts, in elements (rows * cols, or numel):
 * 2^44, about 120 times what one MI355X's 288 GB holds in bfloat16.  The
 * bound keeps every byte offset, index and per-launch count the library
 * forms well inside 64 bits. */
#define NVFP4_MAX_ELEMENTS (INT64_C(1) << 44)

/* Status codes. */
enum {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID = 1,     /* bad argument; nothing launched */
  NVFP4_ERR_UNSUPPORTED = 2, /* valid request the library does not serve */
  NVFP4_ERR_HIP = 3          /* a HIP launch reported an error */
};

/* Block-scale formats.  E4M3 = OCP E4M3FN (bias 7, max 448, 0x7F = NaN).
 * UE5M3 = unsigned, 5 exponent / 3 mantissa bits, bias 15 ("UE5M3" blog,
 * 数学推导 and the emulation in 实现), with subnormals, max 0xFE = 114688
 * and 0xFF = NaN (the E4M3FN conventions carried over). */
enum { NVFP4_SCALE_E4M3 = 0, NVFP4_SCALE_UE5M3 = 1 };

/* Block-scale selection ("Four Over Six" summaries: Methodologie, Key claims;
 * "Scale Learning" blog: the MSE scale sweep that initializes the scales). */
enum {
  NVFP4_SELECT_6 = 0,               /* block max -> 6 */
  NVFP4_SELECT_4OVER6 = 1,          /* max -> 4 or 6, smaller squared error (MSE) */
  NVFP4_SELECT_4OVER6_MAE = 2,      /* max -> 4 or 6, smaller absolute error (MAE) */
  NVFP4_SELECT_4OVER6_MAXERR = 3,   /* max -> 4 or 6, smaller largest error */
  NVFP4_SELECT_SWEEP = 4            /* every scale code, smallest squared error */
};

/* Element rounding: round-to-nearest-even, or stochastic (max->6 only). */
enum { NVFP4_ROUND_RNE = 0, NVFP4_ROUND_SR = 1 };

/* Blocking axes (bitmask): ROW = 16 consecutive elements of a row; COL = 16
 * consecutive rows of a column, written as the row-wise layout of X^T. */
enum { NVFP4_AXIS_ROW = 1, NVFP4_AXIS_COL = 2 };

/* Default FP8 maximum the outer scale maps the tensor amax to. */
#define NVFP4_GLOBAL_MAX_E4M3 448.0f
#define NVFP4_GLOBAL_MAX_E4M3_4OVER6 256.0f
#define NVFP4_GLOBAL_MAX_UE5M3 114688.0f

/* NVFP4_WORKSPACE_BYTES of the loaded library. */
size_t nvfp4_workspace_bytes(void);

/*
 * nvfp4_tensor_amax -- current-tensor scaling: *amax_out = max_i |x_i| over
 * numel bf16 values ("UE5M3" blog, 数学推导: the amax of the whole tensor
 * recomputed at every step).  One launch.
 *   x          device, numel bf16 patterns, 16-byte aligned.
 *   numel      >= 0; 0 writes 0.
 *   amax_out   device, one float; overwritten (no need to clear it).
 *   workspace  a workspace (see above).
 * A NaN anywhere gives NaN; otherwise an infinity gives +inf.
 * Errors: x (numel > 0), amax_out or workspace NULL or misaligned, or
 * numel < 0 or > NVFP4_MAX_ELEMENTS -> NVFP4_ERR_INVALID.
 */
int nvfp4_tensor_amax(const uint16_t* x, int64_t numel, float* amax_out, void* workspace,
                      hipStream_t stream);

/*
 * nvfp4_tensor_amax_noalloc -- nvfp4_tensor_amax without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * workgroups' maxima meet in a static array the library holds on each GPU
 * (NVFP4_WORKSPACE_BYTES per GPU, kept until the process ends); the call
 * allocates nothing.  Every call on one GPU shares that array, so calls that
 * overlap on one GPU (several streams) race; calls in one stream do not.
 * Arguments and result as nvfp4_tensor_amax; any numel.  Errors: as
 * nvfp4_tensor_amax, plus NVFP4_ERR_UNSUPPORTED on a GPU with more than 8192
 * compute units (more workgroups than the array has slots) and
 * NVFP4_ERR_HIP if the array's device address cannot be obtained.
 */
int nvfp4_tensor_amax_noalloc(const uint16_t* x, int64_t numel, float* amax_out,
                              hipStream_t stream);

/*
 * Arguments of the quantize calls: one struct, so that the outputs of the
 * row-wise and column-wise layouts, the optional 4/6 count and its
 * workspace travel together.
 */
typedef struct nvfp4_quant_args {
  const uint16_t* x;            /* bf16 [rows, cols], row-major, 16-byte aligned */
  int64_t rows, cols;
  const float* amax;            /* device: the tensor amax A (one float), or for
                                   nvfp4_quantize_rowscaled one amax per row */
  float global_fp8_max;         /* S_g > 0, or 0 for the default (below) */
  int scale_fmt;                /* NVFP4_SCALE_E4M3 or NVFP4_SCALE_UE5M3 */
  int select;                   /* an NVFP4_SELECT_* rule */
  int rounding;                 /* NVFP4_ROUND_RNE or NVFP4_ROUND_SR */
  int axes;                     /* NVFP4_AXIS_ROW, NVFP4_AXIS_COL or both */
  uint64_t seed;                /* stochastic rounding only */
  uint8_t* codes;               /* ROW: [rows, cols/2], 16-byte aligned */
  uint8_t* scales;              /* ROW: [rows, cols/16], 4-byte aligned */
  uint8_t* codes_t;             /* COL: [cols, rows/2], 16-byte aligned */
  uint8_t* scales_t;            /* COL: [cols, rows/16] */
  unsigned long long* count4;   /* optional: += blocks that chose max->4 */
  void* workspace;              /* required with count4 (see above), else unused */
} nvfp4_quant_args;

/*
 * nvfp4_quantize -- NVFP4 quantization of a bf16 tensor x[rows, cols]: per
 * 16-element block a scale = block amax / 6 encoded to E4M3 under the FP32
 * outer scale, and every element rounded to the E2M1 grid ("End-to-End 4-Bit
 * Training", Low-precision formats on Blackwell; "UE5M3" blog, 数学推导 for
 * the UE5M3 scale); Four-Over-Six also encodes the block with its max
 * mapped to 4 and keeps the lower-error result ("Four Over Six" notes,
 * Method; gist.science summary, Methodologie); stochastic rounding for
 * gradients ("UE5M3" blog, 数学推导; "End-to-End 4-Bit Training",
 * Re-quantization with stochastic rounding); column-wise blocks for the
 * transposed operand ("End-to-End 4-Bit Training", Block-scaled backward
 * passes).  Fields of *args:
 *   amax            the tensor amax A (fresh from nvfp4_tensor_amax, or a
 *                   stale/periodic value, "UE5M3" blog, 数学推导).  The outer
 *                   scale is alpha = A / (6 * global_fp8_max) in binary32
 *                   (alpha = 1 if A = 0).
 *   global_fp8_max  0 selects the default: 448 (E4M3, max->6 and the
 *                   sweep), 256 (E4M3, the Four-Over-Six rules; gist.science
 *                   summary, Implementatiedetails), 114688 (UE5M3).
 *   seed            the variate of the element at index i of the OUTPUT
 *                   orientation (r*cols + c row-wise, c*rows + r column-wise)
 *                   is the counter hash of (seed, i).
 *   count4          += number of blocks (all axes) that chose max->4; the
 *                   caller clears it.  Needs workspace.
 * Per block (binary32, in this order): a = max|x_i|; for Q in {6, 4}:
 * s_raw = a * K_Q with K_Q = 1/(Q*alpha); code = nearest scale code (ties to
 * even, saturating); y_i = x_i * (1/(D[code]*alpha)); E2M1 code of y_i (RNE,
 * or SR); SSE over the block in a fixed 4x4 fmaf tree; max->4 is kept only if
 * its SSE is strictly lower.  With the residuals d_i = fmaf(-q_i, S, x_i):
 * SELECT_4OVER6_MAE compares the sums of |d_i| (the same 4x4 tree, with
 * additions), SELECT_4OVER6_MAXERR the largest |d_i|.  SELECT_SWEEP encodes
 * the block with every finite scale code (ascending) and keeps the one with
 * the strictly smallest SSE (ties keep the smaller code): the MSE scale sweep
 * that initializes scale learning ("Scale Learning" blog); it does not touch
 * count4.
 * A negative or non-finite *amax: every scale byte = the NaN code (0x7F E4M3,
 * 0xFF UE5M3), every element code 0.  A NaN element with a usable amax: same
 * for its block.
 * Errors (NVFP4_ERR_INVALID): args, x or amax NULL; rows or cols < 0; ROW
 * with cols % 16 != 0 or codes/scales NULL; COL with rows % 16 != 0 or
 * codes_t/scales_t NULL; unknown enum; axes == 0; SR with any select but
 * SELECT_6; global_fp8_max negative or non-finite; count4 without workspace;
 * misaligned pointers.  rows == 0 or cols == 0: nothing to do, NVFP4_OK.
 */
int nvfp4_quantize(const nvfp4_quant_args* args, hipStream_t stream);

/*
 * nvfp4_dequantize -- x_hat = q * D[scale code] * alpha, correctly rounded
 * to binary32: the FP4 value times the FP8 block scale times the FP32 outer
 * scale ("End-to-End 4-Bit Training", Low-precision formats on Blackwell);
 * a NaN scale code gives NaN.  Optionally, in the same pass, the squared
 * error against the original tensor, whose mean is the per-tensor MSE and
 * whose square root over ||x|| is the relative error the "UE5M3" blog
 * suggests monitoring (调试指南).
 *   codes, scales   [rows, cols/2], [rows, cols/16] as nvfp4_quantize writes.
 *   amax, global_fp8_max, scale_fmt   as given to nvfp4_quantize; here
 *                   global_fp8_max must be > 0 (the value actually used:
 *                   its default depends on the selection rule, which a
 *                   dequantization does not know).
 *   out_f32         optional [rows, cols] float.
 *   out_bf16        optional [rows, cols] bf16: round-to-nearest-even of the
 *                   binary32 value.
 *   block_scale_out optional [rows, cols/16] float: D * alpha per block (the
 *                   binary32 effective scale; the scale-learning init).
 *   x_ref, sse_out  optional pair: x_ref [rows, cols] bf16 input; *sse_out
 *                   (device double) = sum (x - x_hat)^2, the residual and
 *                   the sum in binary64, combined in a fixed order (the same
 *                   on every run).  Needs workspace.
 *   workspace       required with sse_out (see above), else unused.
 * Errors (NVFP4_ERR_INVALID): codes/scales/amax NULL; rows or cols < 0;
 * cols % 16 != 0; unknown format; global_fp8_max <= 0 or non-finite; exactly
 * one of x_ref / sse_out given; sse_out without workspace; misaligned
 * pointers.
 */
int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                     const float* amax, float global_fp8_max, int scale_fmt, float* out_f32,
                     uint16_t* out_bf16, float* block_scale_out, const uint16_t* x_ref,
                     double* sse_out, void* workspace, hipStream_t stream);

/*
 * nvfp4_fakequant_fwd -- scale-learning fake quantization ("Scale Learning",
 * "How Scale Learning Works"):
 *   x~ = s_post * clamp(round_E2M1(x / s_pre), -6, 6)
 * per 16-element row block b with scales s_pre[b], s_post[b] ([rows, cols/16]
 * floats).  s_post == NULL: tied single scale (s_post = s_pre).
 * x / s_pre is y = x * inv in binary32, inv = 1/s_pre (0 if s_pre = 0,
 * +-FLT_MAX if the reciprocal overflows); x~ = q * s_post rounded once.
 *   xq_out  [rows, cols] float.
 * Errors: NULL x/s_pre/xq_out, rows or cols < 0, cols % 16 != 0, misaligned
 * pointers -> NVFP4_ERR_INVALID.
 */
int nvfp4_fakequant_fwd(const uint16_t* x, int64_t rows, int64_t cols, const float* s_pre,
                        const float* s_post, float* xq_out, hipStream_t stream);

/*
 * nvfp4_fakequant_bwd -- straight-through backward of nvfp4_fakequant_fwd
 * (derivative of round and of the FP8 scale quantization taken as 1).  With
 * in_i = (-6 <= y_i <= 6):
 *  single (s_post == NULL):
 *   grad_x_i   = in_i ? g_i : 0
 *   grad_s_pre = sum_i g_i * (in_i ? q_i - y_i : (y_i < -6 ? -6 : 6))
 *  dual:
 *   grad_x_i    = in_i ? g_i * (s_post / s_pre) : 0   (0 when s_pre = 0)
 *   grad_s_post = sum_i g_i * clamp(q_i)
 *   grad_s_pre  = -(s_post * sum_{in} g_i x_i) / (s_pre * s_pre)  (0 when s_pre = 0)
 * Products and block sums are binary64 (sum in element order) rounded once to
 * binary32, so results do not depend on the launch configuration.
 *   grad_xq      [rows, cols] float, upstream dL/dx~.
 *   grad_x       [rows, cols] float.
 *   grad_s_pre   [rows, cols/16] float (the single-scale gradient when tied).
 *   grad_s_post  [rows, cols/16] float; required for dual, must be NULL when
 *                tied.
 * Errors: as nvfp4_fakequant_fwd, plus grad_s_post presence not matching
 * s_post -> NVFP4_ERR_INVALID.
 */
int nvfp4_fakequant_bwd(const uint16_t* x, const float* grad_xq, int64_t rows, int64_t cols,
                        const float* s_pre, const float* s_post, float* grad_x,
                        float* grad_s_pre, float* grad_s_post, hipStream_t stream);

/*
 * nvfp4_fakequant_fwd_amax / nvfp4_fakequant_bwd_amax -- the same with the
 * trained quantity reparameterized as the block amax ("Scale Learning", How
 * Scale Learning Works: ModelOpt trains amax rather than the scale): per
 * block s_pre = fl(a_pre / 6), s_post = fl(a_post / 6) in binary32, then
 * exactly the scale form; the gradients are with respect to the amaxes,
 * dL/da = dL/ds * ds/da = dL/ds / 6, the division applied to the binary64
 * block sums before their one rounding.  Arguments, layouts and errors as
 * nvfp4_fakequant_fwd / nvfp4_fakequant_bwd with a_* in place of s_*.
 */
int nvfp4_fakequant_fwd_amax(const uint16_t* x, int64_t rows, int64_t cols, const float* a_pre,
                             const float* a_post, float* xq_out, hipStream_t stream);
int nvfp4_fakequant_bwd_amax(const uint16_t* x, const float* grad_xq, int64_t rows, int64_t cols,
                             const float* a_pre, const float* a_post, float* grad_x,
                             float* grad_a_pre, float* grad_a_post, hipStream_t stream);

/* ---------------------------------------------------------------------
 * Per-row outer scales ("End-to-End 4-Bit Training", Recipe details:
 * per-token outer scales when quantizing activations).  Row r has its own
 * FP32 outer scale alpha_r = row_amax[r] / (6 * S_g); every other step is the
 * per-tensor method with A replaced by row_amax[r], so a row's result does
 * not depend on any other row (batch invariance).  A per-expert outer scale
 * is the per-tensor calls applied to each expert's matrix.
 *
 * nvfp4_row_amax -- row_amax[r] = max |x[r, c]| over the row, with the rules
 * of nvfp4_tensor_amax per row (any NaN -> NaN; else an infinity -> +inf; an
 * empty row -> 0).
 *   x         [rows, cols] bf16, 16-byte aligned, cols % 16 == 0.
 *   row_amax  [rows] float, 4-byte aligned; written.
 * Errors: NULL pointers with rows > 0, misalignment, cols % 16 != 0 ->
 * NVFP4_ERR_INVALID.
 */
int nvfp4_row_amax(const uint16_t* x, int64_t rows, int64_t cols, float* row_amax, hipStream_t stream);

/*
 * nvfp4_quantize_rowscaled -- row-wise NVFP4 quantization with per-row
 * outer scales (as nvfp4_quantize with axes = ROW, A_r in place of A).
 *   args->amax  [rows] float on the device (from nvfp4_row_amax, or stale).
 *   args->axes  must be NVFP4_AXIS_ROW.
 *   Other fields and errors as nvfp4_quantize; codes / scales / count4 /
 *   workspace as there.  A row whose amax is negative or non-finite gets the
 *   NaN scale code in every block and element code 0.  SR uses the
 *   row-major element index r * cols + c.
 */
int nvfp4_quantize_rowscaled(const nvfp4_quant_args* args, hipStream_t stream);

/*
 * nvfp4_quantize_pertoken -- per-token quantization: nvfp4_row_amax and
 * then nvfp4_quantize_rowscaled with those amaxes ("End-to-End 4-Bit
 * Training", Recipe details: per-token outer scales), in one launch that
 * reads each row once when cols <= 4096 (longer rows: those two launches).
 *   row_amax_out  [rows] float, 4-byte aligned; written with the row amaxes
 *                 (rules of nvfp4_row_amax), which the quantization uses.
 *   args->amax    not read.  args->axes must be NVFP4_AXIS_ROW.
 *   Other fields, outputs and errors as nvfp4_quantize_rowscaled; the codes,
 *   scales and count4 are bit for bit those of nvfp4_row_amax followed by
 *   nvfp4_quantize_rowscaled.  cols == 0 writes 0 to every row amax.
 */
int nvfp4_quantize_pertoken(const nvfp4_quant_args* args, float* row_amax_out,
                            hipStream_t stream);

/*
 * nvfp4_dequantize_rowscaled -- nvfp4_dequantize with per-row outer scales:
 * x_hat = q * D * alpha_r.  Arguments, outputs and errors as
 * nvfp4_dequantize, with row_amax[rows] in place of amax.
 */
int nvfp4_dequantize_rowscaled(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                               int64_t cols, const float* row_amax, float global_fp8_max,
                               int scale_fmt, float* out_f32, uint16_t* out_bf16,
                               float* block_scale_out, const uint16_t* x_ref, double* sse_out,
                               void* workspace, hipStream_t stream);

/* ---------------------------------------------------------------------
 * nvfp4_quantize_2d -- 16x16 tile scales ("End-to-End 4-Bit Training",
 * Block-scaled backward passes): one block scale per square 16x16 tile, from
 * the tile's amax, shared by the tile's 16 row blocks and 16 column blocks,
 * so the column-wise codes are bit for bit the transpose of the row-wise ones.
 * Max->6 and round-to-nearest-even (the weights path).  Per-tensor outer
 * scale from args->amax as in nvfp4_quantize.  Fields of *args:
 *   x          [rows, cols] bf16, rows % 16 == 0, cols % 16 == 0.
 *   select, rounding  must be NVFP4_SELECT_6 and NVFP4_ROUND_RNE.
 *   axes       NVFP4_AXIS_ROW, or ROW | COL for the transposed layout too.
 *   codes      [rows, cols/2], scales [rows, cols/16] (every row block holds
 *              its tile's code); 16- and 4-byte aligned.
 *   codes_t    [cols, rows/2], scales_t [cols, rows/16]: the layout of X^T
 *              (with COL); codes_t 16-byte aligned.
 *   count4, workspace  unused.
 * NaN rules: a non-finite or negative amax -> NaN scale code everywhere and
 * codes 0; a tile holding a NaN element -> its scale is the NaN code and its
 * codes 0.
 * Errors: NULL / misaligned outputs, shape not a multiple of 16, unknown
 * scale_fmt, another select / rounding, axes without ROW -> NVFP4_ERR_INVALID.
 */
int nvfp4_quantize_2d(const nvfp4_quant_args* args, hipStream_t stream);

/*
 * Re-quantization for the backward pass ("End-to-End 4-Bit Training",
 * Re-quantization with stochastic rounding, and its quantized-linear-layer
 * figure): an NVFP4 tensor saved from the forward pass is dequantized
 * (x_hat = q * D * alpha rounded once to binary32, exactly as
 * nvfp4_dequantize), transposed, and quantized again along the other
 * dimension with stochastic rounding, so that the backward pass sees the
 * forward tensor in expectation.
 *
 * Source (both calls): codes [rows, cols/2] (16-byte aligned), scales
 * [rows, cols/16] (2-byte aligned), scale_fmt and its S_g = global_fp8_max (> 0, the value
 * the tensor was quantized with), and exactly one of amax (one device float:
 * per-tensor outer scale) and row_amax ([rows] device floats: per-row outer
 * scales, as nvfp4_quantize_rowscaled).  cols % 16 == 0.
 */
enum { NVFP4_TARGET_NVFP4 = 0, NVFP4_TARGET_MXFP8 = 1 };

/*
 * nvfp4_dequantized_amax -- *amax_out = max |x_hat| over the tensor (the
 * current amax of the dequantized tensor, for the outer scale of an NVFP4
 * re-quantization); NaN if any x_hat is NaN.  amax_out 4-byte aligned;
 * workspace as for nvfp4_tensor_amax.  One launch.
 * Errors: NULL or misaligned pointers, both or neither of amax / row_amax,
 * cols % 16 != 0, unknown scale_fmt, global_fp8_max not > 0 ->
 * NVFP4_ERR_INVALID.
 */
int nvfp4_dequantized_amax(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                           const float* amax, const float* row_amax, float global_fp8_max,
                           int scale_fmt, float* amax_out, void* workspace, hipStream_t stream);

/*
 * nvfp4_requantize_t -- quantize X_hat^T ([cols, rows], row-major) with
 * stochastic rounding.  The SR variate of an element is the hash of its
 * index in X_hat^T, c * rows + r, under `seed` (as nvfp4_quantize).
 *   target NVFP4_TARGET_NVFP4: max->6, E2M1 with SR, outer scale from
 *     *dst_amax (device float; e.g. from nvfp4_dequantized_amax, or the
 *     source amax) with S_g = dst_global_fp8_max (0 -> the max->6 default of
 *     dst_scale_fmt).  rows % 16 == 0.  out_t = codes [cols, rows/2]
 *     (16-byte aligned), out_scales_t = scales [cols, rows/16].
 *   target NVFP4_TARGET_MXFP8 (OCP Microscaling, the pages' backward
 *     format): blocks of 32 source rows of one column; E8M0 scale byte
 *     e + 127 with e = floor(log2 amax_b) - 8 (at least -127); elements
 *     x_hat * 2^-e clamped to +-448 and rounded onto E4M3 with SR
 *     (round up iff (h >> 12) + floor(2^20 p) >= 2^20).  rows % 32 == 0.
 *     out_t = E4M3 bytes [cols, rows] (16-byte aligned), out_scales_t =
 *     E8M0 bytes [cols, rows/32].  dst_amax, dst_global_fp8_max and
 *     dst_scale_fmt are ignored.
 * NaN rules: a NaN x_hat makes its output block's scale the NaN code (0x7F /
 * 0xFF for NVFP4, 0xFF for MXFP8) and the block's elements 0; so does an
 * infinite x_hat for MXFP8 (its E8M0 exponent is not representable); a
 * negative or non-finite *dst_amax gives NaN scale codes everywhere (NVFP4).
 * Errors: as nvfp4_dequantized_amax, plus unknown target or dst_scale_fmt,
 * rows not a multiple of the target's block, NULL or misaligned outputs ->
 * NVFP4_ERR_INVALID.
 */
int nvfp4_requantize_t(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                       const float* amax, const float* row_amax, float global_fp8_max,
                       int scale_fmt, int target, const float* dst_amax, float dst_global_fp8_max,
                       int dst_scale_fmt, uint64_t seed, uint8_t* out_t, uint8_t* out_scales_t,
                       hipStream_t stream);

/*
 * 16-point random Hadamard transform around quantization ("Four Over Six"
 * notes, Method: NVIDIA's recipe applies it to both inputs of the weight-
 * gradient GEMM; "End-to-End 4-Bit Training", Quantized communications: an
 * orthogonal rotation that spreads outliers and is inverted exactly).  Per
 * NVFP4 block (16 consecutive elements of a row for axis ROW, 16 consecutive
 * rows of a column for axis COL):
 *   y = H16 diag(s) x / 4,
 * H16 the Sylvester Hadamard matrix, s_j = -1 iff the top bit of the counter
 * hash of (sign_seed, j) is set (one sign vector per tensor), computed in
 * binary32 as x_j * (+-0.25) followed by the fast Walsh-Hadamard butterfly
 * (stages 1, 2, 4, 8; (a, b) -> (a + b, a - b)).  The inverse scales by
 * 0.25, runs the same butterfly and applies the signs.
 *
 * nvfp4_rht_amax -- *amax_out = max |y| over the transformed tensor (the
 * outer amax for nvfp4_quantize_rht; NaN if any element is NaN).  x [rows,
 * cols] bf16; ROW: cols % 16 == 0, x 16-byte aligned; COL: rows % 16 == 0.
 * workspace as for nvfp4_tensor_amax.  One launch.
 *
 * nvfp4_quantize_rht -- nvfp4_quantize of the transformed tensor, along one
 * axis (args->axes = NVFP4_AXIS_ROW or NVFP4_AXIS_COL, not both): ROW writes
 * codes [rows, cols/2] and scales [rows, cols/16]; COL writes the column-wise
 * layout (of the transpose) into codes_t [cols, rows/2] and scales_t [cols,
 * rows/16].  Other fields as nvfp4_quantize (SR indices in the output
 * orientation).
 *
 * nvfp4_dequantize_rht -- x_hat of an NVFP4 tensor [rows, cols] (as
 * nvfp4_dequantize), then the inverse transform of every 16-element row
 * block: out_f32 [rows, cols] (16-byte aligned).  For a COL-quantized
 * tensor pass its layout ([cols, rows]); the result is then the transpose.
 * Errors: NULL or misaligned pointers, shapes not multiples of 16 along the
 * blocked axis, unknown enums, SR with a select other than SELECT_6 ->
 * NVFP4_ERR_INVALID.
 */
int nvfp4_rht_amax(const uint16_t* x, int64_t rows, int64_t cols, int axis, uint64_t sign_seed,
                   float* amax_out, void* workspace, hipStream_t stream);
int nvfp4_quantize_rht(const nvfp4_quant_args* args, uint64_t sign_seed, hipStream_t stream);
int nvfp4_dequantize_rht(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                         const float* amax, float global_fp8_max, int scale_fmt,
                         uint64_t sign_seed, float* out_f32, hipStream_t stream);

/* Static description of a status code. */
const char* nvfp4_status_string(int status);

/* NVFP4_ABI_VERSION of the loaded library. */
int nvfp4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
