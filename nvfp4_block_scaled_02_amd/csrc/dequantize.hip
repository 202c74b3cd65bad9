// dequantize.hip -- NVFP4 -> binary32 / bf16 ("End-to-End 4-Bit Training",
// "Low-precision formats on Blackwell": value = fp4 x fp8 x fp32).
//
// x_hat = (q * D) * alpha: q * D is exact in binary32 (2 + 4 significant
// bits), so the second product is the correctly rounded q * D * alpha.  q
// comes from the exact hardware E2M1 decode.  Optionally the same pass reads
// the bf16 input and accumulates sum (x - x_hat)^2 in binary64 (the per-tensor
// error report).  HBM-bound: 0.5625 B read + 4 (2) B written per element,
// plus 2 B read with the error report.
#include "common.hpp"
#include "device.hpp"

namespace nvfp4 {

constexpr int kDqUnroll = 2;

__device__ __forceinline__ double wave_sum_f64(double v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int FMT, bool F32, bool BF16, bool BSC, bool SSE>
__global__ void __launch_bounds__(kThreads)
dequantize_kernel(const uint32_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                  int64_t nchunks, const float* __restrict__ amax, float sg,
                  float4* __restrict__ out_f32, uint4* __restrict__ out_bf16,
                  float* __restrict__ block_scale, const uint4* __restrict__ x_ref,
                  double* sse) {
  const TensorScale ts = tensor_scale(*amax, sg);
  const float alpha = ts.nan ? __builtin_nanf("") : ts.alpha;
  const bool even = (threadIdx.x & 1) == 0;
  double acc = 0.0;
  const int64_t per_iter = (int64_t)gridDim.x * kThreads * kDqUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kDqUnroll; base < nchunks; base += per_iter) {
    uint32_t cw[kDqUnroll];
    uint32_t sc[kDqUnroll];
    uint4 xr[kDqUnroll];
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
      const int64_t ch = base + u * kThreads + threadIdx.x;
      const bool ok = ch < nchunks;
      cw[u] = ok ? ld_nt(codes + ch) : 0u;
      sc[u] = ok ? (uint32_t)scales[ch >> 1] : 0u;
      if (SSE) xr[u] = ok ? ld_nt(x_ref + ch) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
      const int64_t ch = base + u * kThreads + threadIdx.x;
      if (ch >= nchunks) continue;
      const float D = decode_scale(FMT, sc[u]);
      float q[8], v[8];
      e2m1_unpack8(cw[u], q);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (q[i] * D) * alpha;
      if (F32) {
        st_nt(make_float4(v[0], v[1], v[2], v[3]), out_f32 + 2 * ch);
        st_nt(make_float4(v[4], v[5], v[6], v[7]), out_f32 + 2 * ch + 1);
      }
      if (BF16) {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t b = __float_as_uint(v[i]);
          const uint32_t r = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
          h[i] = v[i] != v[i] ? ((b >> 16) | 0x40u) : r;
        }
        st_nt(make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                               h[4] | (h[5] << 16), h[6] | (h[7] << 16)),
                                    out_bf16 + ch);
      }
      if (BSC && even) block_scale[ch >> 1] = D * alpha;
      if (SSE) {
        const float xs[8] = {bf16_lo(xr[u].x), bf16_hi(xr[u].x), bf16_lo(xr[u].y), bf16_hi(xr[u].y),
                             bf16_lo(xr[u].z), bf16_hi(xr[u].z), bf16_lo(xr[u].w), bf16_hi(xr[u].w)};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double d = (double)xs[i] - (double)v[i];
          acc += d * d;
        }
      }
    }
  }
  if (SSE) {
    __shared__ double red[kThreads / 64];
    acc = wave_sum_f64(acc);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
      double t = 0.0;
      for (int i = 0; i < kThreads / 64; ++i) t += red[i];
      unsafeAtomicAdd(sse, t);
    }
  }
}

template <int FMT, bool F32, bool BF16, bool BSC, bool SSE>
static hipError_t launch_dq(const DequantizeArgs& a, hipStream_t s) {
  const int64_t nchunks = a.rows * a.cols / kChunk;
  const int64_t per_wg = (int64_t)kThreads * kDqUnroll;
  int64_t grid = (nchunks + per_wg - 1) / per_wg;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  grid = grid < cap ? grid : cap;
  hipLaunchKernelGGL((dequantize_kernel<FMT, F32, BF16, BSC, SSE>), dim3((unsigned)grid),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint32_t*>(a.codes), a.scales,
                     nchunks, a.amax, a.sg, reinterpret_cast<float4*>(a.out_f32),
                     reinterpret_cast<uint4*>(a.out_bf16), a.block_scale,
                     reinterpret_cast<const uint4*>(a.x_ref), a.sse);
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
