// common.hpp -- definitions shared by the host entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

enum { FMT_E4M3 = 0, FMT_UE5M3 = 1 };
// block-scale selection: max->6; Four-Over-Six by squared error, absolute
// error or largest error; or the smallest squared error over every code
enum { SELECT_6 = 0, SELECT_4OVER6 = 1, SELECT_4OVER6_MAE = 2, SELECT_4OVER6_MAXERR = 3,
       SELECT_SWEEP = 4 };
constexpr bool is_four_six(int select) { return select >= SELECT_4OVER6 && select <= SELECT_4OVER6_MAXERR; }
enum { ROUND_RNE = 0, ROUND_SR = 1 };
enum { AXIS_ROW = 1, AXIS_COL = 2 };

// Launch shape of the streaming kernels: 256 threads = 4 wave64s per
// workgroup; each lane owns 8 consecutive elements (one 16-byte bf16 chunk)
// and two neighbouring lanes own one 16-element block.
constexpr int kThreads = 256;
constexpr int kChunk = 8;

struct QuantizeArgs {
  const uint16_t* x;
  int64_t rows, cols;
  const float* amax;
  float sg;  // resolved S_g (> 0)
  int fmt, select, rounding, axes;
  uint64_t seed;
  uint8_t *codes, *scales, *codes_t, *scales_t;
  unsigned long long* count4;
  uint8_t* ws;  // workspace of the count's grid reduction (with count4)
};

struct DequantizeArgs {
  const uint8_t *codes, *scales;
  int64_t rows, cols;
  const float* amax;
  float sg;
  int fmt;
  float* out_f32;
  uint16_t* out_bf16;
  float* block_scale;
  const uint16_t* x_ref;
  double* sse;
  uint8_t* ws;      // workspace of the error report's grid reduction (with sse)
  bool row_scaled;  // amax points to one amax per row (per-row outer scales)
};

struct FakeQuantArgs {
  const uint16_t* x;
  const float* g;
  int64_t rows, cols;
  const float *s_pre, *s_post;
  float* xq;
  float *dx, *ds_pre, *ds_post;
  bool amax_param;  // s_pre / s_post hold amaxes (s = a / 6); gradients w.r.t. them
};

// Re-quantization of an NVFP4 tensor: dequantize, transpose, quantize again
// with stochastic rounding (target 0 = NVFP4, 1 = MXFP8).
struct RequantArgs {
  const uint8_t *codes, *scales;  // source [rows, cols/2], [rows, cols/16]
  int64_t rows, cols;
  const float* amax;      // per-tensor outer amax, or nullptr
  const float* row_amax;  // one outer amax per row, or nullptr
  float sg;               // resolved S_g of the source
  int fmt;                // source scale format
  int target;
  const float* dst_amax;  // NVFP4 target: outer amax of the re-quantized tensor
  float dst_sg;
  int dst_fmt;
  uint64_t seed;
  uint8_t *out_t, *out_scales_t;
};

// Launchers (one translation unit each); return the hipError_t of the launch.
// Launchers taking `ws` reduce one value per workgroup in that workspace
// (grid_reduce.hpp: kWorkspaceBytes, counters zero on entry and on exit).
hipError_t launch_tensor_amax(const uint16_t* x, int64_t numel, float* out, uint8_t* ws,
                              hipStream_t s);
hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t s);
hipError_t launch_row_amax(const uint16_t* x, int64_t rows, int64_t cols, float* out, hipStream_t s);
// a.amax = one amax per row
hipError_t launch_quantize_rowscaled(const QuantizeArgs& a, hipStream_t s);
// the row amaxes computed in the same launch and written to row_amax_out
// (a.amax unused), then as launch_quantize_rowscaled
hipError_t launch_quantize_pertoken(const QuantizeArgs& a, float* row_amax_out, hipStream_t s);
// 16x16 tile scales (max->6, RNE); a.axes = ROW or ROW | COL
hipError_t launch_quantize_2d(const QuantizeArgs& a, hipStream_t s);
hipError_t launch_dequantize(const DequantizeArgs& a, hipStream_t s);
// every block transformed by the 16-point random Hadamard transform with sign
// mask `signs` first; a.axes = ROW or COL
hipError_t launch_quantize_rht(const QuantizeArgs& a, uint32_t signs, hipStream_t s);
// amax of the transformed tensor (axis ROW or COL), and dequantize + inverse
hipError_t launch_rht_amax(const uint16_t* x, int64_t rows, int64_t cols, int axis, uint32_t signs,
                           float* out, uint8_t* ws, hipStream_t s);
hipError_t launch_dequantize_rht(const DequantizeArgs& a, uint32_t signs, hipStream_t s);
hipError_t launch_fakequant_fwd(const FakeQuantArgs& a, hipStream_t s);
hipError_t launch_fakequant_bwd(const FakeQuantArgs& a, hipStream_t s);
hipError_t launch_requant_t(const RequantArgs& a, hipStream_t s);
hipError_t launch_dequantized_amax(const RequantArgs& a, float* out, uint8_t* ws, hipStream_t s);
// test hook: E4M3 SR element bytes through the re-quantizer's packing routine
hipError_t launch_test_e4m3_sr(const float* y, const uint32_t* h, int64_t n, uint8_t* codes,
                               hipStream_t s);

// Number of compute units of the current device (cached per device).
int device_cu_count();

}  // namespace nvfp4
