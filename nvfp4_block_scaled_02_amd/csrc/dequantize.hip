// dequantize.hip -- NVFP4 -> binary32 / bf16 ("End-to-End 4-Bit Training",
// "Low-precision formats on Blackwell": value = fp4 x fp8 x fp32; per-row
// fp32 outer scales: Recipe details).
//
// x_hat = (q * D) * alpha: q * D is exact in binary32 (2 + 4 significant
// bits), so the second product is the correctly rounded q * D * alpha.  q
// comes from the exact hardware E2M1 decode.  Optionally the same pass reads
// the bf16 input and accumulates sum (x - x_hat)^2 in binary64 (the per-tensor
// error report).  HBM-bound: 0.5625 B read + 4 (2) B written per element,
// plus 2 B read with the error report.
#include "common.hpp"
#include "device.hpp"
#include "grid_reduce.hpp"

namespace nvfp4 {

// Mapping: a lane owns 4 consecutive elements (2 code bytes) so that every
// load and store instruction of a wavefront covers contiguous memory (one
// float4 store per lane for binary32 output); 4 lanes share a block's scale
// byte.  Outputs use non-temporal stores.
//
// Error report: the residual x - x_hat is taken in binary64 (exact unless x
// is more than 2^29 times x_hat, i.e. a block scale saturated far below its
// data), squared and accumulated in binary64 per
// lane in a fixed order; the workgroups' sums meet in the caller's workspace
// and the last workgroup adds them in index order (grid_reduce.hpp), so the
// report is the same on every run of a launch shape.
constexpr int kDqUnroll = 4;

__device__ __forceinline__ uint32_t bf16_rne(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t r = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
  return v != v ? ((b >> 16) | 0x40u) : r;
}

template <int FMT, bool F32, bool BF16, bool BSC, bool SSE, int BLOCK>
__global__ void __launch_bounds__(BLOCK)
dequantize_kernel(const uint16_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                  int64_t nquads, const float* __restrict__ amax, float sg,
                  float4* __restrict__ out_f32, uint2* __restrict__ out_bf16,
                  float* __restrict__ block_scale, const uint2* __restrict__ x_ref,
                  double* sse, uint8_t* ws) {
  const bool lead4 = (threadIdx.x & 3) == 0;
  double acc = 0.0;
  const int64_t per_iter = (int64_t)gridDim.x * BLOCK * kDqUnroll;
  uint32_t cw[kDqUnroll], sc[kDqUnroll];
  uint2 xr[kDqUnroll];
  auto load = [&](int64_t base) {
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
      const int64_t qd = base + u * BLOCK + threadIdx.x;
      const bool ok = qd < nquads;
      cw[u] = ok ? (uint32_t)codes[qd] : 0u;
      sc[u] = ok ? (uint32_t)scales[qd >> 2] : 0u;
      if (SSE) xr[u] = ok ? ld_nt(x_ref + qd) : make_uint2(0, 0);
    }
  };
  // The first trip's loads go out before the outer scale is read (two
  // dependent scalar loads and a division), so their latency overlaps it;
  // each later trip's loads are issued at the end of the one before.
  int64_t base = (int64_t)blockIdx.x * BLOCK * kDqUnroll;
  load(base);
  const float alpha = outer_alpha(*amax, sg);
  for (; base < nquads; base += per_iter) {
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
      const int64_t qd = base + u * BLOCK + threadIdx.x;
      if (qd >= nquads) continue;
      const float D = decode_scale(FMT, sc[u]);
      const f32x2 q01 = NVFP4_DEC_PK_FP4(cw[u], 0), q23 = NVFP4_DEC_PK_FP4(cw[u], 1);
      const float v[4] = {(q01[0] * D) * alpha, (q01[1] * D) * alpha, (q23[0] * D) * alpha,
                          (q23[1] * D) * alpha};
      if (F32) st_nt(make_float4(v[0], v[1], v[2], v[3]), out_f32 + qd);
      if (BF16) {
        const uint2 h = make_uint2(bf16_rne(v[0]) | (bf16_rne(v[1]) << 16),
                                   bf16_rne(v[2]) | (bf16_rne(v[3]) << 16));
        st_nt(h, out_bf16 + qd);
      }
      if (BSC && lead4) block_scale[qd >> 2] = D * alpha;
      if (SSE) {
        const float xs[4] = {bf16_lo(xr[u].x), bf16_hi(xr[u].x), bf16_lo(xr[u].y), bf16_hi(xr[u].y)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const double d = (double)xs[i] - (double)v[i];
          acc = __builtin_fma(d, d, acc);
        }
      }
    }
    if (base + per_iter < nquads) load(base + per_iter);
  }
  if constexpr (SSE) {
    double total;
    if (grid_reduce<SumF64, BLOCK>(ws, acc, &total)) *sse = total;
  }
}

// Per-row outer scales: a workgroup owns whole rows, kDqUnroll of them at a
// time (rows r, r + G, r + 2G, ... for G = grid size), forms each row's
// alpha_r once, and lane t handles quad t (then t + BLOCK, ...) of each of
// those rows, so every lane keeps kDqUnroll independent loads in flight
// whatever the row length.
template <int FMT, bool F32, bool BF16, bool BSC, bool SSE, int BLOCK>
__global__ void __launch_bounds__(BLOCK)
dequantize_rows_kernel(const uint16_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                       int64_t rows, int64_t qpr, const float* __restrict__ row_amax, float sg,
                       float4* __restrict__ out_f32, uint2* __restrict__ out_bf16,
                       float* __restrict__ block_scale, const uint2* __restrict__ x_ref,
                       double* sse, uint8_t* ws) {
  const bool lead4 = (threadIdx.x & 3) == 0;
  const int64_t G = gridDim.x;
  double acc = 0.0;
  for (int64_t r0 = blockIdx.x; r0 < rows; r0 += G * kDqUnroll) {
    float alpha[kDqUnroll];
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
      const int64_t r = r0 + u * G;
      alpha[u] = r < rows ? outer_alpha(row_amax[r], sg) : 0.0f;
    }
    for (int64_t q = threadIdx.x; q < qpr; q += BLOCK) {
      uint32_t cw[kDqUnroll], sc[kDqUnroll];
      uint2 xr[kDqUnroll];
#pragma unroll
      for (int u = 0; u < kDqUnroll; ++u) {
        const int64_t r = r0 + u * G;
        const bool ok = r < rows;
        const int64_t qd = r * qpr + q;
        cw[u] = ok ? (uint32_t)codes[qd] : 0u;
        sc[u] = ok ? (uint32_t)scales[qd >> 2] : 0u;
        if (SSE) xr[u] = ok ? ld_nt(x_ref + qd) : make_uint2(0, 0);
      }
#pragma unroll
      for (int u = 0; u < kDqUnroll; ++u) {
        const int64_t r = r0 + u * G;
        if (r >= rows) continue;
        const int64_t qd = r * qpr + q;
        const float D = decode_scale(FMT, sc[u]);
        const f32x2 q01 = NVFP4_DEC_PK_FP4(cw[u], 0), q23 = NVFP4_DEC_PK_FP4(cw[u], 1);
        const float v[4] = {(q01[0] * D) * alpha[u], (q01[1] * D) * alpha[u],
                            (q23[0] * D) * alpha[u], (q23[1] * D) * alpha[u]};
        if (F32) st_nt(make_float4(v[0], v[1], v[2], v[3]), out_f32 + qd);
        if (BF16) {
          const uint2 h = make_uint2(bf16_rne(v[0]) | (bf16_rne(v[1]) << 16),
                                     bf16_rne(v[2]) | (bf16_rne(v[3]) << 16));
          st_nt(h, out_bf16 + qd);
        }
        if (BSC && lead4) block_scale[qd >> 2] = D * alpha[u];
        if (SSE) {
          const float xs[4] = {bf16_lo(xr[u].x), bf16_hi(xr[u].x), bf16_lo(xr[u].y), bf16_hi(xr[u].y)};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const double d = (double)xs[i] - (double)v[i];
            acc = __builtin_fma(d, d, acc);
          }
        }
      }
    }
  }
  if constexpr (SSE) {
    double total;
    if (grid_reduce<SumF64, BLOCK>(ws, acc, &total)) *sse = total;
  }
}

template <int FMT, bool F32, bool BF16, bool BSC, bool SSE>
static hipError_t launch_dq(const DequantizeArgs& a, hipStream_t s) {
  constexpr int BLOCK = SSE ? 1024 : kThreads;
  const int64_t cus = device_cu_count();
  if (a.row_scaled) {
    // SSE: one 1024-lane workgroup per CU (88 registers: two do not fit)
    int64_t cap = cus * (SSE ? 1 : 8);
    cap = cap < kSlots ? cap : kSlots;
    const int64_t grid = a.rows < cap ? a.rows : cap;
    hipLaunchKernelGGL((dequantize_rows_kernel<FMT, F32, BF16, BSC, SSE, BLOCK>),
                       dim3((unsigned)grid), dim3(BLOCK), 0, s,
                       reinterpret_cast<const uint16_t*>(a.codes), a.scales, a.rows, a.cols / 4,
                       a.amax, a.sg, reinterpret_cast<float4*>(a.out_f32),
                       reinterpret_cast<uint2*>(a.out_bf16), a.block_scale,
                       reinterpret_cast<const uint2*>(a.x_ref), a.sse, a.ws);
    return hipGetLastError();
  }
  // SSE: two 1024-lane workgroups per CU (8 wavefronts per SIMD): 39.5 us
  // at 8192x4096 against 42.1 with one, four give 40.0
  int64_t cap = cus * (SSE ? 2 : 8);
  cap = cap < kSlots ? cap : kSlots;
  const int64_t nquads = a.rows * a.cols / 4;
  const int64_t per_wg = (int64_t)BLOCK * kDqUnroll;
  int64_t grid = (nquads + per_wg - 1) / per_wg;
  grid = grid < cap ? grid : cap;
  hipLaunchKernelGGL((dequantize_kernel<FMT, F32, BF16, BSC, SSE, BLOCK>), dim3((unsigned)grid),
                     dim3(BLOCK), 0, s, reinterpret_cast<const uint16_t*>(a.codes), a.scales,
                     nquads, a.amax, a.sg, reinterpret_cast<float4*>(a.out_f32),
                     reinterpret_cast<uint2*>(a.out_bf16), a.block_scale,
                     reinterpret_cast<const uint2*>(a.x_ref), a.sse, a.ws);
  return hipGetLastError();
}

template <int FMT, bool F32, bool BF16, bool BSC>
static hipError_t launch_dq3(const DequantizeArgs& a, hipStream_t s) {
  return a.sse ? launch_dq<FMT, F32, BF16, BSC, true>(a, s) : launch_dq<FMT, F32, BF16, BSC, false>(a, s);
}
template <int FMT, bool F32, bool BF16>
static hipError_t launch_dq2(const DequantizeArgs& a, hipStream_t s) {
  return a.block_scale ? launch_dq3<FMT, F32, BF16, true>(a, s) : launch_dq3<FMT, F32, BF16, false>(a, s);
}
template <int FMT, bool F32>
static hipError_t launch_dq1(const DequantizeArgs& a, hipStream_t s) {
  return a.out_bf16 ? launch_dq2<FMT, F32, true>(a, s) : launch_dq2<FMT, F32, false>(a, s);
}
template <int FMT>
static hipError_t launch_dq0(const DequantizeArgs& a, hipStream_t s) {
  return a.out_f32 ? launch_dq1<FMT, true>(a, s) : launch_dq1<FMT, false>(a, s);
}

hipError_t launch_dequantize(const DequantizeArgs& a, hipStream_t s) {
  return a.fmt == FMT_E4M3 ? launch_dq0<FMT_E4M3>(a, s) : launch_dq0<FMT_UE5M3>(a, s);
}

}  // namespace nvfp4
