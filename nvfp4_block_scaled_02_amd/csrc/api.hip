// api.hip -- the extern "C" entry points of libnvfp4.so (include/nvfp4.h):
// host-side validation, resolution of defaults, and dispatch to the kernels.
// Nothing here allocates device memory or synchronizes.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/nvfp4.h"
#include "../../include/nvfp4_testing.h"
#include "common.hpp"
#include "device.hpp"
#include "grid_reduce.hpp"

namespace nvfp4 {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static bool size_ok(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return false;
  if (cols != 0 && rows > NVFP4_MAX_ELEMENTS / cols) return false;
  return true;
}

static int status_of(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

// ---------------------------------------------------------------- test hooks
__global__ void test_e2m1_range_kernel(uint32_t first, int64_t n, uint8_t* codes) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float y = __uint_as_float(first + (uint32_t)i);
    codes[i] = (uint8_t)(NVFP4_CVT_PK_FP4(0u, y, 0.0f, 0) & 0xFu);
  }
}

// Eight values per thread through the quantizer's own packing routine (so
// both nibble positions of the instruction are exercised); n % 8 == 0.
__global__ void test_e2m1_sr_kernel(const float* y, const uint32_t* h, int64_t n, uint8_t* codes) {
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n / 8;
       g += (int64_t)gridDim.x * blockDim.x) {
    f32x2 yp[4];
    uint32_t hh[8];
    for (int b = 0; b < 4; ++b) yp[b] = f32x2{y[8 * g + 2 * b], y[8 * g + 2 * b + 1]};
    for (int i = 0; i < 8; ++i) hh[i] = h[8 * g + i];
    const uint32_t w = e2m1_sr_pack8(yp, hh, 0u, 0u);
    for (int i = 0; i < 8; ++i) codes[8 * g + i] = (uint8_t)((w >> (4 * i)) & 0xFu);
  }
}

template <int FMT>
__global__ void test_scale_range_kernel(uint32_t first, int64_t n, uint8_t* codes) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float s = __uint_as_float(first + (uint32_t)i);
    codes[i] = (uint8_t)(encode_pair(FMT, s, 0.0f) & 0xFFu);
  }
}

__global__ void test_sr_hash_kernel(uint64_t seed, uint64_t idx0, int64_t n, uint32_t key0,
                                    uint32_t* out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint64_t idx = idx0 + (uint64_t)i;
    const uint32_t hi = (uint32_t)(idx >> 32);
    const uint32_t key = hi == 0 ? key0 : sr_key(seed, hi);
    out[i] = fmix32((uint32_t)idx ^ key);
  }
}

static unsigned test_grid(int64_t n) {
  int64_t g = (n + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 16;
  return (unsigned)(g < 1 ? 1 : (g < cap ? g : cap));
}

// ---------------------------------------------------------------- static scratch
// The workspace of nvfp4_tensor_amax_noalloc: one array per GPU, in the
// library's own device memory (it is zero at load, like every static object,
// and every call that completes leaves its counters zero again).  Host code
// never uses the array's name as an address: the device address of each
// GPU's copy comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[kWorkspaceBytes];

constexpr int kMaxDevices = 64;
static std::atomic<uint8_t*> g_scratch[kMaxDevices];
static std::mutex g_scratch_mu;

// Device address of the current device's scratch, or nullptr.
static uint8_t* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  uint8_t* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr)
      return nullptr;
    p = static_cast<uint8_t*>(addr);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" {

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_INVALID: return "invalid argument";
    case NVFP4_ERR_UNSUPPORTED: return "unsupported request";
    case NVFP4_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

static_assert(NVFP4_WORKSPACE_BYTES == kWorkspaceBytes, "header and kernels agree on the workspace");

size_t nvfp4_workspace_bytes(void) { return kWorkspaceBytes; }

static float resolve_sg(float global_fp8_max, int scale_fmt, int select) {
  if (global_fp8_max != 0.0f) return global_fp8_max;
  if (scale_fmt == NVFP4_SCALE_UE5M3) return NVFP4_GLOBAL_MAX_UE5M3;
  return (select >= NVFP4_SELECT_4OVER6 && select <= NVFP4_SELECT_4OVER6_MAXERR)
             ? NVFP4_GLOBAL_MAX_E4M3_4OVER6 : NVFP4_GLOBAL_MAX_E4M3;
}

static bool ws_ok(const void* ws) { return ws != nullptr && aligned16(ws); }

int nvfp4_tensor_amax(const uint16_t* x, int64_t numel, float* amax_out, void* workspace,
                      hipStream_t stream) {
  if (numel < 0 || numel > NVFP4_MAX_ELEMENTS || !amax_out || !ws_ok(workspace))
    return NVFP4_ERR_INVALID;
  if (numel > 0 && (!x || !aligned16(x))) return NVFP4_ERR_INVALID;
  if (((uintptr_t)amax_out & 3u) != 0) return NVFP4_ERR_INVALID;
  return status_of(launch_tensor_amax(x, numel, amax_out, static_cast<uint8_t*>(workspace), stream));
}

int nvfp4_tensor_amax_noalloc(const uint16_t* x, int64_t numel, float* amax_out,
                              hipStream_t stream) {
  if (numel < 0 || numel > NVFP4_MAX_ELEMENTS || !amax_out) return NVFP4_ERR_INVALID;
  if (numel > 0 && (!x || !aligned16(x))) return NVFP4_ERR_INVALID;
  if (((uintptr_t)amax_out & 3u) != 0) return NVFP4_ERR_INVALID;
  // the kernel's grid (one workgroup per CU at most) must fit the scratch's slots
  if (device_cu_count() > kSlots) return NVFP4_ERR_UNSUPPORTED;
  uint8_t* ws = scratch_of_current_device();
  if (!ws) return NVFP4_ERR_HIP;
  return status_of(launch_tensor_amax(x, numel, amax_out, ws, stream));
}

// Checks shared by the quantize calls; fills the kernel-side arguments.
static int quant_common(const nvfp4_quant_args* p, QuantizeArgs& a) {
  if (!p || !p->x || !p->amax || !size_ok(p->rows, p->cols)) return NVFP4_ERR_INVALID;
  if (p->scale_fmt != NVFP4_SCALE_E4M3 && p->scale_fmt != NVFP4_SCALE_UE5M3) return NVFP4_ERR_INVALID;
  if (p->select < NVFP4_SELECT_6 || p->select > NVFP4_SELECT_SWEEP) return NVFP4_ERR_INVALID;
  if (p->rounding != NVFP4_ROUND_RNE && p->rounding != NVFP4_ROUND_SR) return NVFP4_ERR_INVALID;
  if (p->rounding == NVFP4_ROUND_SR && p->select != NVFP4_SELECT_6) return NVFP4_ERR_INVALID;
  if (p->axes != NVFP4_AXIS_ROW && p->axes != NVFP4_AXIS_COL &&
      p->axes != (NVFP4_AXIS_ROW | NVFP4_AXIS_COL))
    return NVFP4_ERR_INVALID;
  if (!(p->global_fp8_max >= 0.0f) || isinf(p->global_fp8_max)) return NVFP4_ERR_INVALID;
  if (p->axes & NVFP4_AXIS_ROW) {
    if (p->cols % 16 != 0 || !p->codes || !p->scales || !aligned16(p->codes) ||
        ((uintptr_t)p->scales & 3u))
      return NVFP4_ERR_INVALID;
  }
  if (p->axes & NVFP4_AXIS_COL) {
    if (p->rows % 16 != 0 || p->cols % 8 != 0 || !p->codes_t || !p->scales_t || !aligned16(p->codes_t))
      return NVFP4_ERR_INVALID;
  }
  if (!aligned16(p->x) || ((uintptr_t)p->amax & 3u) || ((uintptr_t)p->count4 & 7u))
    return NVFP4_ERR_INVALID;
  if (p->count4 && !ws_ok(p->workspace)) return NVFP4_ERR_INVALID;
  a.x = p->x; a.rows = p->rows; a.cols = p->cols; a.amax = p->amax;
  a.sg = resolve_sg(p->global_fp8_max, p->scale_fmt, p->select);
  a.fmt = p->scale_fmt; a.select = p->select; a.rounding = p->rounding; a.axes = p->axes;
  a.seed = p->seed;
  a.codes = (p->axes & NVFP4_AXIS_ROW) ? p->codes : nullptr;
  a.scales = (p->axes & NVFP4_AXIS_ROW) ? p->scales : nullptr;
  a.codes_t = (p->axes & NVFP4_AXIS_COL) ? p->codes_t : nullptr;
  a.scales_t = (p->axes & NVFP4_AXIS_COL) ? p->scales_t : nullptr;
  a.count4 = p->count4;
  a.ws = p->count4 ? static_cast<uint8_t*>(p->workspace) : nullptr;
  return NVFP4_OK;
}

int nvfp4_quantize(const nvfp4_quant_args* args, hipStream_t stream) {
  QuantizeArgs a;
  const int st = quant_common(args, a);
  if (st != NVFP4_OK) return st;
  if (a.rows == 0 || a.cols == 0) return NVFP4_OK;
  return status_of(launch_quantize(a, stream));
}

static int dq_common(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                     const float* amax, float global_fp8_max, int scale_fmt, float* out_f32,
                     uint16_t* out_bf16, float* block_scale_out, const uint16_t* x_ref,
                     double* sse_out, void* workspace, bool row_scaled, DequantizeArgs& a) {
  if (!codes || !scales || !amax || !size_ok(rows, cols) || cols % 16 != 0) return NVFP4_ERR_INVALID;
  if (scale_fmt != NVFP4_SCALE_E4M3 && scale_fmt != NVFP4_SCALE_UE5M3) return NVFP4_ERR_INVALID;
  if (!(global_fp8_max > 0.0f) || isinf(global_fp8_max)) return NVFP4_ERR_INVALID;
  if ((x_ref == nullptr) != (sse_out == nullptr)) return NVFP4_ERR_INVALID;
  if (sse_out && !ws_ok(workspace)) return NVFP4_ERR_INVALID;
  if (!aligned16(codes) || !aligned16(out_f32) || !aligned16(out_bf16) || !aligned16(x_ref))
    return NVFP4_ERR_INVALID;
  if (((uintptr_t)amax & 3u) || ((uintptr_t)block_scale_out & 3u) || ((uintptr_t)sse_out & 7u))
    return NVFP4_ERR_INVALID;
  a.codes = codes; a.scales = scales; a.rows = rows; a.cols = cols; a.amax = amax;
  a.sg = global_fp8_max; a.fmt = scale_fmt; a.out_f32 = out_f32; a.out_bf16 = out_bf16;
  a.block_scale = block_scale_out; a.x_ref = x_ref; a.sse = sse_out;
  a.ws = sse_out ? static_cast<uint8_t*>(workspace) : nullptr; a.row_scaled = row_scaled;
  return NVFP4_OK;
}

int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                     const float* amax, float global_fp8_max, int scale_fmt, float* out_f32,
                     uint16_t* out_bf16, float* block_scale_out, const uint16_t* x_ref,
                     double* sse_out, void* workspace, hipStream_t stream) {
  DequantizeArgs a;
  const int st = dq_common(codes, scales, rows, cols, amax, global_fp8_max, scale_fmt, out_f32,
                           out_bf16, block_scale_out, x_ref, sse_out, workspace, false, a);
  if (st != NVFP4_OK) return st;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  return status_of(launch_dequantize(a, stream));
}

int nvfp4_row_amax(const uint16_t* x, int64_t rows, int64_t cols, float* row_amax, hipStream_t stream) {
  if (!size_ok(rows, cols) || cols % 16 != 0) return NVFP4_ERR_INVALID;
  if (rows > 0 && (!x || !row_amax || !aligned16(x) || ((uintptr_t)row_amax & 3u)))
    return NVFP4_ERR_INVALID;
  if (rows == 0) return NVFP4_OK;
  return status_of(launch_row_amax(x, rows, cols, row_amax, stream));
}

int nvfp4_quantize_rowscaled(const nvfp4_quant_args* args, hipStream_t stream) {
  if (!args || args->axes != NVFP4_AXIS_ROW) return NVFP4_ERR_INVALID;
  QuantizeArgs a;
  const int st = quant_common(args, a);
  if (st != NVFP4_OK) return st;
  if (a.rows == 0 || a.cols == 0) return NVFP4_OK;
  return status_of(launch_quantize_rowscaled(a, stream));
}

int nvfp4_quantize_pertoken(const nvfp4_quant_args* args, float* row_amax_out,
                            hipStream_t stream) {
  if (!args || args->axes != NVFP4_AXIS_ROW) return NVFP4_ERR_INVALID;
  if (!row_amax_out || ((uintptr_t)row_amax_out & 3u)) return NVFP4_ERR_INVALID;
  nvfp4_quant_args p = *args;
  p.amax = row_amax_out;  // args->amax is not read
  QuantizeArgs a;
  const int st = quant_common(&p, a);
  if (st != NVFP4_OK) return st;
  if (a.rows == 0) return NVFP4_OK;
  // empty rows: their amaxes (0) are the whole output
  if (a.cols == 0) return status_of(launch_row_amax(a.x, a.rows, 0, row_amax_out, stream));
  return status_of(launch_quantize_pertoken(a, row_amax_out, stream));
}

int nvfp4_dequantize_rowscaled(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                               int64_t cols, const float* row_amax, float global_fp8_max,
                               int scale_fmt, float* out_f32, uint16_t* out_bf16,
                               float* block_scale_out, const uint16_t* x_ref, double* sse_out,
                               void* workspace, hipStream_t stream) {
  DequantizeArgs a;
  const int st = dq_common(codes, scales, rows, cols, row_amax, global_fp8_max, scale_fmt, out_f32,
                           out_bf16, block_scale_out, x_ref, sse_out, workspace, true, a);
  if (st != NVFP4_OK) return st;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  return status_of(launch_dequantize(a, stream));
}

int nvfp4_quantize_2d(const nvfp4_quant_args* args, hipStream_t stream) {
  if (!args) return NVFP4_ERR_INVALID;
  const nvfp4_quant_args* p = args;
  if (!p->x || !p->amax || !size_ok(p->rows, p->cols) || p->rows % 16 != 0 || p->cols % 16 != 0)
    return NVFP4_ERR_INVALID;
  if (p->scale_fmt != NVFP4_SCALE_E4M3 && p->scale_fmt != NVFP4_SCALE_UE5M3) return NVFP4_ERR_INVALID;
  if (p->select != NVFP4_SELECT_6 || p->rounding != NVFP4_ROUND_RNE) return NVFP4_ERR_INVALID;
  if (p->axes != NVFP4_AXIS_ROW && p->axes != (NVFP4_AXIS_ROW | NVFP4_AXIS_COL)) return NVFP4_ERR_INVALID;
  if (!(p->global_fp8_max >= 0.0f) || isinf(p->global_fp8_max)) return NVFP4_ERR_INVALID;
  if (!p->codes || !p->scales || !aligned16(p->codes) || ((uintptr_t)p->scales & 3u))
    return NVFP4_ERR_INVALID;
  const bool both = p->axes & NVFP4_AXIS_COL;
  if (both && (!p->codes_t || !p->scales_t || !aligned16(p->codes_t))) return NVFP4_ERR_INVALID;
  if (!aligned16(p->x) || ((uintptr_t)p->amax & 3u)) return NVFP4_ERR_INVALID;
  if (p->rows == 0 || p->cols == 0) return NVFP4_OK;
  QuantizeArgs a;
  a.x = p->x; a.rows = p->rows; a.cols = p->cols; a.amax = p->amax;
  a.sg = resolve_sg(p->global_fp8_max, p->scale_fmt, NVFP4_SELECT_6);
  a.fmt = p->scale_fmt; a.select = SELECT_6; a.rounding = ROUND_RNE;
  a.axes = both ? (AXIS_ROW | AXIS_COL) : AXIS_ROW; a.seed = 0;
  a.codes = p->codes; a.scales = p->scales;
  a.codes_t = both ? p->codes_t : nullptr; a.scales_t = both ? p->scales_t : nullptr;
  a.count4 = nullptr; a.ws = nullptr;
  return status_of(launch_quantize_2d(a, stream));
}

static int rq_source(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                     const float* amax, const float* row_amax, float global_fp8_max,
                     int scale_fmt) {
  if (!codes || !scales || !size_ok(rows, cols) || cols % 16 != 0) return NVFP4_ERR_INVALID;
  if ((amax == nullptr) == (row_amax == nullptr)) return NVFP4_ERR_INVALID;
  if (scale_fmt != NVFP4_SCALE_E4M3 && scale_fmt != NVFP4_SCALE_UE5M3) return NVFP4_ERR_INVALID;
  if (!(global_fp8_max > 0.0f) || isinf(global_fp8_max)) return NVFP4_ERR_INVALID;
  if (!aligned16(codes) || ((uintptr_t)scales & 1u) || ((uintptr_t)amax & 3u) ||
      ((uintptr_t)row_amax & 3u))
    return NVFP4_ERR_INVALID;
  return NVFP4_OK;
}

int nvfp4_dequantized_amax(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                           const float* amax, const float* row_amax, float global_fp8_max,
                           int scale_fmt, float* amax_out, void* workspace, hipStream_t stream) {
  const int st = rq_source(codes, scales, rows, cols, amax, row_amax, global_fp8_max, scale_fmt);
  if (st != NVFP4_OK) return st;
  if (!amax_out || ((uintptr_t)amax_out & 3u) || !ws_ok(workspace)) return NVFP4_ERR_INVALID;
  RequantArgs a = {};
  a.codes = codes; a.scales = scales; a.rows = rows; a.cols = cols;
  a.amax = amax; a.row_amax = row_amax; a.sg = global_fp8_max; a.fmt = scale_fmt;
  return status_of(launch_dequantized_amax(a, amax_out, static_cast<uint8_t*>(workspace), stream));
}

int nvfp4_requantize_t(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                       const float* amax, const float* row_amax, float global_fp8_max,
                       int scale_fmt, int target, const float* dst_amax, float dst_global_fp8_max,
                       int dst_scale_fmt, uint64_t seed, uint8_t* out_t, uint8_t* out_scales_t,
                       hipStream_t stream) {
  const int st = rq_source(codes, scales, rows, cols, amax, row_amax, global_fp8_max, scale_fmt);
  if (st != NVFP4_OK) return st;
  if (!out_t || !out_scales_t || !aligned16(out_t)) return NVFP4_ERR_INVALID;
  if (target == NVFP4_TARGET_NVFP4) {
    if (rows % 16 != 0 || !dst_amax || ((uintptr_t)dst_amax & 3u)) return NVFP4_ERR_INVALID;
    if (dst_scale_fmt != NVFP4_SCALE_E4M3 && dst_scale_fmt != NVFP4_SCALE_UE5M3)
      return NVFP4_ERR_INVALID;
    if (!(dst_global_fp8_max >= 0.0f) || isinf(dst_global_fp8_max)) return NVFP4_ERR_INVALID;
  } else if (target == NVFP4_TARGET_MXFP8) {
    if (rows % 32 != 0) return NVFP4_ERR_INVALID;
  } else {
    return NVFP4_ERR_INVALID;
  }
  if (rows == 0 || cols == 0) return NVFP4_OK;
  RequantArgs a = {};
  a.codes = codes; a.scales = scales; a.rows = rows; a.cols = cols;
  a.amax = amax; a.row_amax = row_amax; a.sg = global_fp8_max; a.fmt = scale_fmt;
  a.target = target; a.seed = seed; a.out_t = out_t; a.out_scales_t = out_scales_t;
  if (target == NVFP4_TARGET_NVFP4) {
    a.dst_amax = dst_amax; a.dst_fmt = dst_scale_fmt;
    a.dst_sg = resolve_sg(dst_global_fp8_max, dst_scale_fmt, NVFP4_SELECT_6);
  } else {
    a.dst_amax = nullptr; a.dst_fmt = FMT_E4M3; a.dst_sg = 0.0f;
  }
  return status_of(launch_requant_t(a, stream));
}

// ---------------------------------------------------------------- random Hadamard transform
// Sign mask of the tensor: bit j set iff the top bit of the counter hash of
// (sign_seed, j) is set.
static uint32_t rht_signs(uint64_t sign_seed) {
  const uint32_t k = sr_key(sign_seed, 0u);
  uint32_t m = 0;
  for (uint32_t j = 0; j < 16; ++j)
    if (fmix32(j ^ k) >> 31) m |= 1u << j;
  return m;
}

int nvfp4_rht_amax(const uint16_t* x, int64_t rows, int64_t cols, int axis, uint64_t sign_seed,
                   float* amax_out, void* workspace, hipStream_t stream) {
  if (!x || !amax_out || !size_ok(rows, cols) || ((uintptr_t)amax_out & 3u)) return NVFP4_ERR_INVALID;
  if (!ws_ok(workspace)) return NVFP4_ERR_INVALID;
  if (axis == NVFP4_AXIS_ROW) {
    if (cols % 16 != 0 || !aligned16(x)) return NVFP4_ERR_INVALID;
  } else if (axis == NVFP4_AXIS_COL) {
    if (rows % 16 != 0 || ((uintptr_t)x & 1u)) return NVFP4_ERR_INVALID;
  } else {
    return NVFP4_ERR_INVALID;
  }
  return status_of(launch_rht_amax(x, rows, cols, axis, rht_signs(sign_seed), amax_out,
                                   static_cast<uint8_t*>(workspace), stream));
}

int nvfp4_quantize_rht(const nvfp4_quant_args* args, uint64_t sign_seed, hipStream_t stream) {
  if (!args || (args->axes != NVFP4_AXIS_ROW && args->axes != NVFP4_AXIS_COL)) return NVFP4_ERR_INVALID;
  QuantizeArgs a;
  const int st = quant_common(args, a);
  if (st != NVFP4_OK) return st;
  if (a.rows == 0 || a.cols == 0) return NVFP4_OK;
  return status_of(launch_quantize_rht(a, rht_signs(sign_seed), stream));
}

int nvfp4_dequantize_rht(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                         const float* amax, float global_fp8_max, int scale_fmt,
                         uint64_t sign_seed, float* out_f32, hipStream_t stream) {
  if (!codes || !scales || !amax || !out_f32 || !size_ok(rows, cols) || cols % 16 != 0)
    return NVFP4_ERR_INVALID;
  if (scale_fmt != NVFP4_SCALE_E4M3 && scale_fmt != NVFP4_SCALE_UE5M3) return NVFP4_ERR_INVALID;
  if (!(global_fp8_max > 0.0f) || isinf(global_fp8_max)) return NVFP4_ERR_INVALID;
  if (((uintptr_t)codes & 7u) || !aligned16(out_f32) || ((uintptr_t)amax & 3u))
    return NVFP4_ERR_INVALID;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  DequantizeArgs a = {};
  a.codes = codes; a.scales = scales; a.rows = rows; a.cols = cols; a.amax = amax;
  a.sg = global_fp8_max; a.fmt = scale_fmt; a.out_f32 = out_f32;
  return status_of(launch_dequantize_rht(a, rht_signs(sign_seed), stream));
}

static int fq_common(const uint16_t* x, int64_t rows, int64_t cols, const float* s_pre) {
  if (!x || !s_pre || !size_ok(rows, cols) || cols % 16 != 0) return NVFP4_ERR_INVALID;
  if (!aligned16(x) || ((uintptr_t)s_pre & 3u)) return NVFP4_ERR_INVALID;
  return NVFP4_OK;
}

static int fq_fwd(const uint16_t* x, int64_t rows, int64_t cols, const float* s_pre,
                  const float* s_post, float* xq_out, bool amax_param, hipStream_t stream) {
  int st = fq_common(x, rows, cols, s_pre);
  if (st != NVFP4_OK) return st;
  if (!xq_out || !aligned16(xq_out) || ((uintptr_t)s_post & 3u)) return NVFP4_ERR_INVALID;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  FakeQuantArgs a = {};
  a.x = x; a.rows = rows; a.cols = cols; a.s_pre = s_pre; a.s_post = s_post; a.xq = xq_out;
  a.amax_param = amax_param;
  return status_of(launch_fakequant_fwd(a, stream));
}

static int fq_bwd(const uint16_t* x, const float* grad_xq, int64_t rows, int64_t cols,
                  const float* s_pre, const float* s_post, float* grad_x, float* grad_s_pre,
                  float* grad_s_post, bool amax_param, hipStream_t stream) {
  int st = fq_common(x, rows, cols, s_pre);
  if (st != NVFP4_OK) return st;
  if (!grad_xq || !grad_x || !grad_s_pre) return NVFP4_ERR_INVALID;
  if ((s_post == nullptr) != (grad_s_post == nullptr)) return NVFP4_ERR_INVALID;
  if (!aligned16(grad_xq) || !aligned16(grad_x) || ((uintptr_t)grad_s_pre & 3u) ||
      ((uintptr_t)s_post & 3u) || ((uintptr_t)grad_s_post & 3u))
    return NVFP4_ERR_INVALID;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  FakeQuantArgs a = {};
  a.x = x; a.g = grad_xq; a.rows = rows; a.cols = cols; a.s_pre = s_pre; a.s_post = s_post;
  a.dx = grad_x; a.ds_pre = grad_s_pre; a.ds_post = grad_s_post; a.amax_param = amax_param;
  return status_of(launch_fakequant_bwd(a, stream));
}

int nvfp4_fakequant_fwd(const uint16_t* x, int64_t rows, int64_t cols, const float* s_pre,
                        const float* s_post, float* xq_out, hipStream_t stream) {
  return fq_fwd(x, rows, cols, s_pre, s_post, xq_out, false, stream);
}

int nvfp4_fakequant_bwd(const uint16_t* x, const float* grad_xq, int64_t rows, int64_t cols,
                        const float* s_pre, const float* s_post, float* grad_x,
                        float* grad_s_pre, float* grad_s_post, hipStream_t stream) {
  return fq_bwd(x, grad_xq, rows, cols, s_pre, s_post, grad_x, grad_s_pre, grad_s_post, false,
                stream);
}

int nvfp4_fakequant_fwd_amax(const uint16_t* x, int64_t rows, int64_t cols, const float* a_pre,
                             const float* a_post, float* xq_out, hipStream_t stream) {
  return fq_fwd(x, rows, cols, a_pre, a_post, xq_out, true, stream);
}

int nvfp4_fakequant_bwd_amax(const uint16_t* x, const float* grad_xq, int64_t rows, int64_t cols,
                             const float* a_pre, const float* a_post, float* grad_x,
                             float* grad_a_pre, float* grad_a_post, hipStream_t stream) {
  return fq_bwd(x, grad_xq, rows, cols, a_pre, a_post, grad_x, grad_a_pre, grad_a_post, true,
                stream);
}

// ---------------------------------------------------------------- test hooks
int nvfp4_test_e2m1_rne_range(uint32_t first, int64_t n, uint8_t* codes, hipStream_t stream) {
  if (n < 0 || n > (INT64_C(1) << 32) || (uint64_t)first + (uint64_t)n > (UINT64_C(1) << 32) ||
      (n > 0 && !codes))
    return NVFP4_ERR_INVALID;
  if (n == 0) return NVFP4_OK;
  hipLaunchKernelGGL(test_e2m1_range_kernel, dim3(test_grid(n)), dim3(256), 0,
                     stream, first, n, codes);
  return status_of(hipGetLastError());
}

int nvfp4_test_e2m1_sr(const float* y, const uint32_t* h, int64_t n, uint8_t* codes, hipStream_t stream) {
  if (n < 0 || n % 8 != 0 || (n > 0 && (!y || !h || !codes))) return NVFP4_ERR_INVALID;
  if (n == 0) return NVFP4_OK;
  hipLaunchKernelGGL(test_e2m1_sr_kernel, dim3(test_grid(n / 8)), dim3(256), 0,
                     stream, y, h, n, codes);
  return status_of(hipGetLastError());
}

int nvfp4_test_scale_encode_range(int fmt, uint32_t first, int64_t n, uint8_t* codes,
                                  hipStream_t stream) {
  if (fmt != NVFP4_SCALE_E4M3 && fmt != NVFP4_SCALE_UE5M3) return NVFP4_ERR_INVALID;
  if (n < 0 || (uint64_t)first + (uint64_t)n > (UINT64_C(1) << 31) || (n > 0 && !codes))
    return NVFP4_ERR_INVALID;
  if (n == 0) return NVFP4_OK;
  if (fmt == NVFP4_SCALE_E4M3)
    hipLaunchKernelGGL(test_scale_range_kernel<FMT_E4M3>, dim3(test_grid(n)), dim3(256), 0,
                       stream, first, n, codes);
  else
    hipLaunchKernelGGL(test_scale_range_kernel<FMT_UE5M3>, dim3(test_grid(n)), dim3(256), 0,
                       stream, first, n, codes);
  return status_of(hipGetLastError());
}

int nvfp4_test_e4m3_sr(const float* y, const uint32_t* h, int64_t n, uint8_t* codes, hipStream_t stream) {
  if (n < 0 || n % 4 != 0 || (n > 0 && (!y || !h || !codes))) return NVFP4_ERR_INVALID;
  if (n == 0) return NVFP4_OK;
  return status_of(launch_test_e4m3_sr(y, h, n, codes, stream));
}

int nvfp4_test_sr_hash(uint64_t seed, uint64_t idx0, int64_t n, uint32_t* out, hipStream_t stream) {
  if (n < 0 || (n > 0 && !out)) return NVFP4_ERR_INVALID;
  if (n == 0) return NVFP4_OK;
  hipLaunchKernelGGL(test_sr_hash_kernel, dim3(test_grid(n)), dim3(256), 0, stream,
                     seed, idx0, n, sr_key(seed, 0u), out);
  return status_of(hipGetLastError());
}

}  // extern "C"
