// amax.hip -- tensor amax for current-tensor scaling ("UE5M3: 给 FP4 训练算
// 一笔更宽容的账", section 数学推导): A = max |x| over a bf16 tensor.
//
// HBM-bound (2 bytes read per element).  One 1024-thread workgroup per CU;
// each lane streams 16-byte chunks with non-temporal loads, four in flight,
// folding them with packed 16-bit integer max on the sign-cleared patterns
// (integer order = magnitude order; NaN > inf > finite).  The workgroups'
// maxima meet in the caller's workspace (grid_reduce.hpp): the last
// workgroup to finish writes the float whose bits are (pattern << 16).  One
// launch, nothing to clear beforehand.
#include "common.hpp"
#include "device.hpp"
#include "grid_reduce.hpp"

namespace nvfp4 {

constexpr int kAmaxUnroll = 4;
constexpr int kAmaxThreads = 1024;

__global__ void __launch_bounds__(kAmaxThreads) amax_kernel(const uint4* __restrict__ x, int64_t nchunks,
                                                        const uint16_t* __restrict__ tail,
                                                        int ntail, float* __restrict__ out,
                                                        uint8_t* __restrict__ ws) {
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kAmaxThreads;
  int64_t i = (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x;
  // unrolled body: kAmaxUnroll independent 16-byte loads in flight per lane
  for (; i + (kAmaxUnroll - 1) * stride < nchunks; i += kAmaxUnroll * stride) {
    uint4 w[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) w[u] = ld_nt(x + i + u * stride);
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      uint32_t v = chunk_abs_max_bits(w[u]);
      m = m > v ? m : v;
    }
  }
  for (; i < nchunks; i += stride) {
    uint32_t v = chunk_abs_max_bits(ld_nt(x + i));
    m = m > v ? m : v;
  }
  if (blockIdx.x == 0 && threadIdx.x < ntail) {
    uint32_t v = tail[threadIdx.x] & 0x7FFFu;
    m = m > v ? m : v;
  }
  uint32_t r;
  if (grid_reduce<MaxU32, kAmaxThreads>(ws, m, &r)) out[0] = __uint_as_float(r << 16);
}

// Per-row amax (per-token outer scales, "End-to-End 4-Bit Training", Recipe
// details).  A wavefront owns whole rows: its lanes stream the row's 16-byte
// chunks (four in flight), fold them with the same packed 16-bit integer max
// on sign-cleared patterns, reduce across the wavefront and lane 0 stores the
// row's float.  No atomics.  cols % 16 == 0, so a row is whole chunks.
constexpr int kRowAmaxUnroll = 4;

__global__ void __launch_bounds__(kThreads) row_amax_kernel(const uint4* __restrict__ x, int64_t rows,
                                                           int64_t row_chunks, float* __restrict__ out) {
  const int l = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); r < rows; r += nwaves) {
    const uint4* xr = x + r * row_chunks;
    uint32_t m = 0;
    int64_t i = l;
    for (; i + (kRowAmaxUnroll - 1) * 64 < row_chunks; i += kRowAmaxUnroll * 64) {
      uint4 w[kRowAmaxUnroll];
#pragma unroll
      for (int u = 0; u < kRowAmaxUnroll; ++u) w[u] = ld_nt(xr + i + u * 64);
#pragma unroll
      for (int u = 0; u < kRowAmaxUnroll; ++u) {
        const uint32_t v = chunk_abs_max_bits(w[u]);
        m = m > v ? m : v;
      }
    }
    for (; i < row_chunks; i += 64) {
      const uint32_t v = chunk_abs_max_bits(ld_nt(xr + i));
      m = m > v ? m : v;
    }
    m = wave_reduce<MaxU32>(m);
    if (l == 0) out[r] = __uint_as_float(m << 16);
  }
}

hipError_t launch_row_amax(const uint16_t* x, int64_t rows, int64_t cols, float* out, hipStream_t s) {
  const int64_t per_wg = kThreads / 64;  // rows in flight per workgroup
  int64_t grid = (rows + per_wg - 1) / per_wg;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  grid = grid < cap ? grid : cap;
  hipLaunchKernelGGL(row_amax_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s,
                     reinterpret_cast<const uint4*>(x), rows, cols / kChunk, out);
  return hipGetLastError();
}

hipError_t launch_tensor_amax(const uint16_t* x, int64_t numel, float* out, uint8_t* ws,
                              hipStream_t s) {
  const int64_t nchunks = numel / kChunk;
  const int ntail = (int)(numel - nchunks * kChunk);
  // one workgroup per CU (fewer if the tensor is small); an empty tensor
  // runs one workgroup, which writes 0
  const int64_t want = (nchunks + (int64_t)kAmaxThreads * kAmaxUnroll - 1) / ((int64_t)kAmaxThreads * kAmaxUnroll);
  const int64_t cap = (int64_t)device_cu_count() < kSlots ? (int64_t)device_cu_count() : kSlots;
  int64_t grid = want < cap ? want : cap;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)grid), dim3(kAmaxThreads), 0, s,
                     reinterpret_cast<const uint4*>(x), nchunks, x + nchunks * kChunk, ntail, out, ws);
  return hipGetLastError();
}

}  // namespace nvfp4
