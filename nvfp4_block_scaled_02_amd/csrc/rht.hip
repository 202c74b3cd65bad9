// rht.hip -- the 16-point random Hadamard transform around NVFP4 quantization
// on gfx950 ("Four Over Six" notes, Method: applied to both inputs of the
// weight-gradient GEMM; "End-to-End 4-Bit Training", Quantized
// communications: an orthogonal rotation that spreads outliers and is
// inverted exactly): the amax of the transformed tensor (the outer scale of
// its quantization), and dequantization followed by the inverse transform.
// The quantization of the transformed tensor itself is in quantize.hip (the
// transform runs in registers inside the block quantizers).
#include "grid_reduce.hpp"
#include "quantize_core.hpp"

namespace nvfp4 {

constexpr int kRhtThreads = 1024;
constexpr int kRhtUnroll = 2;

// The grid maximum of the per-lane maxima m (sign-cleared binary32 patterns)
// written to *out by the last workgroup (grid_reduce.hpp).
__device__ __forceinline__ void rht_amax_flush(uint32_t m, float* out, uint8_t* ws) {
  uint32_t r;
  if (grid_reduce<MaxU32, kRhtThreads>(ws, m, &r)) out[0] = __uint_as_float(r);
}

// Largest sign-cleared binary32 pattern of a transformed block (NaN beats
// infinity beats every finite value).
__device__ __forceinline__ uint32_t block_max_bits(const float (&y)[16]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t b = __float_as_uint(y[i]) & 0x7FFFFFFFu;
    m = m > b ? m : b;
  }
  return m;
}

// Row blocks: a lane transforms whole blocks (two 16-byte chunks).
__global__ void __launch_bounds__(kRhtThreads)
rht_amax_rows_kernel(const uint4* __restrict__ x, int64_t nblocks, uint32_t signs,
                     float* __restrict__ out, uint8_t* __restrict__ ws) {
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kRhtThreads;
  int64_t i = (int64_t)blockIdx.x * kRhtThreads + threadIdx.x;
  for (; i + (kRhtUnroll - 1) * stride < nblocks; i += kRhtUnroll * stride) {
    uint4 a[kRhtUnroll], b[kRhtUnroll];
#pragma unroll
    for (int u = 0; u < kRhtUnroll; ++u) {
      a[u] = ld_nt(x + 2 * (i + u * stride));
      b[u] = ld_nt(x + 2 * (i + u * stride) + 1);
    }
#pragma unroll
    for (int u = 0; u < kRhtUnroll; ++u) {
      float y[16];
      unpack16(a[u], b[u], y);
      rht16(y, signs);
      const uint32_t v = block_max_bits(y);
      m = m > v ? m : v;
    }
  }
  for (; i < nblocks; i += stride) {
    float y[16];
    unpack16(ld_nt(x + 2 * i), ld_nt(x + 2 * i + 1), y);
    rht16(y, signs);
    const uint32_t v = block_max_bits(y);
    m = m > v ? m : v;
  }
  rht_amax_flush(m, out, ws);
}

// Column blocks: a lane transforms the 16 values of one column in one group
// of 16 rows.  With cols % 4 == 0 a lane takes four adjacent columns (16
// loads of 8 bytes, 512 contiguous bytes per wavefront load); otherwise one
// column (16 loads of one bf16).
__global__ void __launch_bounds__(kRhtThreads)
rht_amax_cols4_kernel(const uint2* __restrict__ x, int64_t rows, int64_t quads, uint32_t signs,
                      float* __restrict__ out, uint8_t* __restrict__ ws) {
  uint32_t m = 0;
  const int64_t items = (rows / 16) * quads;
  const bool narrow = (items >> 32) == 0;
  const int64_t stride = (int64_t)gridDim.x * kRhtThreads;
  for (int64_t w = (int64_t)blockIdx.x * kRhtThreads + threadIdx.x; w < items; w += stride) {
    const int64_t g = narrow ? (int64_t)((uint32_t)w / (uint32_t)quads) : w / quads;
    const int64_t q = w - g * quads;
    const uint2* p = x + g * 16 * quads + q;
    uint2 v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = ld_nt(p + r * quads);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float y[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t wd = k < 2 ? v[r].x : v[r].y;
        y[r] = (k & 1) ? bf16_hi(wd) : bf16_lo(wd);
      }
      rht16(y, signs);
      const uint32_t b = block_max_bits(y);
      m = m > b ? m : b;
    }
  }
  rht_amax_flush(m, out, ws);
}

__global__ void __launch_bounds__(kRhtThreads)
rht_amax_cols_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, uint32_t signs,
                     float* __restrict__ out, uint8_t* __restrict__ ws) {
  uint32_t m = 0;
  const int64_t items = (rows / 16) * cols;
  const bool narrow = (items >> 32) == 0;
  const int64_t stride = (int64_t)gridDim.x * kRhtThreads;
  for (int64_t w = (int64_t)blockIdx.x * kRhtThreads + threadIdx.x; w < items; w += stride) {
    const int64_t g = narrow ? (int64_t)((uint32_t)w / (uint32_t)cols) : w / cols;
    const int64_t c = w - g * cols;
    const uint16_t* p = x + g * 16 * cols + c;
    float y[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) y[r] = __uint_as_float((uint32_t)p[r * cols] << 16);
    rht16(y, signs);
    const uint32_t v = block_max_bits(y);
    m = m > v ? m : v;
  }
  rht_amax_flush(m, out, ws);
}

hipError_t launch_rht_amax(const uint16_t* x, int64_t rows, int64_t cols, int axis, uint32_t signs,
                           float* out, uint8_t* ws, hipStream_t s) {
  const int64_t items = axis == AXIS_ROW ? rows * cols / 16 : (rows / 16) * cols;
  // one workgroup per CU at most (an empty tensor runs one, which writes 0)
  int64_t cap = (int64_t)device_cu_count();
  cap = cap < kSlots ? cap : kSlots;
  int64_t grid = (items + kRhtThreads - 1) / kRhtThreads;
  grid = grid < cap ? grid : cap;
  if (grid < 1) grid = 1;
  if (axis == AXIS_ROW) {
    hipLaunchKernelGGL(rht_amax_rows_kernel, dim3((unsigned)grid), dim3(kRhtThreads), 0, s,
                       reinterpret_cast<const uint4*>(x), items, signs, out, ws);
  } else if (cols % 4 == 0 && ((uintptr_t)x & 7u) == 0) {
    const int64_t quads = cols / 4;
    int64_t g4 = ((rows / 16) * quads + kRhtThreads - 1) / kRhtThreads;
    g4 = g4 < cap ? g4 : cap;
    if (g4 < 1) g4 = 1;
    hipLaunchKernelGGL(rht_amax_cols4_kernel, dim3((unsigned)g4), dim3(kRhtThreads), 0, s,
                       reinterpret_cast<const uint2*>(x), rows, quads, signs, out, ws);
  } else {
    hipLaunchKernelGGL(rht_amax_cols_kernel, dim3((unsigned)grid), dim3(kRhtThreads), 0, s, x, rows,
                       cols, signs, out, ws);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- dequantize + inverse
// A lane per block: x_hat = (q * D) * alpha (as the dequantize kernel) and
// the inverse transform in registers.  Stores go through the wavefront's LDS: lane l holds block (g*64 + l)'s 64
// bytes; after the bounce lane l writes float4 l + 64k of the group's 4 KiB,
// so every store instruction writes 1 KiB contiguous.  Blocks are taken in
// whole wavefront groups (a partial last group stores only its blocks).
template <int FMT>
__global__ void __launch_bounds__(kThreads)
dequantize_rht_kernel(const uint2* __restrict__ codes, const uint8_t* __restrict__ scales,
                      int64_t nblocks, const float* __restrict__ amax, float sg, uint32_t signs,
                      float4* __restrict__ out) {
  __shared__ float4 bounce[kThreads * 4];
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
  float4* reg = bounce + wv * 256;
  const float alpha = outer_alpha(*amax, sg);
  const int64_t ngroups = (nblocks + 63) / 64;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t g = (int64_t)blockIdx.x * (kThreads / 64) + wv; g < ngroups; g += nwaves) {
    const int64_t i = g * 64 + l;
    const bool ok = i < nblocks;
    const uint2 w = ok ? ld_nt(codes + i) : make_uint2(0, 0);
    const float D = ok ? decode_scale(FMT, scales[i]) : 0.0f;
    float q[16], v[16];
    float qa[8], qb[8];
    e2m1_unpack8(w.x, qa);
    e2m1_unpack8(w.y, qb);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      q[e] = qa[e];
      q[8 + e] = qb[e];
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = (q[e] * D) * alpha;
    irht16(v, signs);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int k = 0; k < 4; ++k) reg[4 * l + k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t f0 = g * 256;                       // first float4 of the group
    const int64_t fend = nblocks * 4;                 // float4s in the tensor
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t f = f0 + l + 64 * k;
      if (f < fend) st_nt(reg[l + 64 * k], out + f);
    }
  }
}

hipError_t launch_dequantize_rht(const DequantizeArgs& a, uint32_t signs, hipStream_t s) {
  const int64_t nblocks = a.rows * a.cols / 16;
  int64_t grid = ((nblocks + 63) / 64 + kThreads / 64 - 1) / (kThreads / 64);
  const int64_t cap = (int64_t)device_cu_count() * 8;
  grid = grid < cap ? grid : cap;
  if (a.fmt == FMT_UE5M3)
    hipLaunchKernelGGL(dequantize_rht_kernel<FMT_UE5M3>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                       reinterpret_cast<const uint2*>(a.codes), a.scales, nblocks, a.amax, a.sg,
                       signs, reinterpret_cast<float4*>(a.out_f32));
  else
    hipLaunchKernelGGL(dequantize_rht_kernel<FMT_E4M3>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                       reinterpret_cast<const uint2*>(a.codes), a.scales, nblocks, a.amax, a.sg,
                       signs, reinterpret_cast<float4*>(a.out_f32));
  return hipGetLastError();
}

}  // namespace nvfp4
