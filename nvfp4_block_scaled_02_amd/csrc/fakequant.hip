// fakequant.hip -- scale-learning fake quantization and its straight-through
// gradients ("Scale Learning: Training NVFP4 Block Scales to Recover
// Accuracy", section "How Scale Learning Works").
//
// Forward: x~ = s_post * clamp(round_E2M1(x / s_pre), -6, 6) per 16-element
// row block; x / s_pre is y = x * (1 / s_pre) in binary32 and the E2M1
// rounding is the hardware conversion (round-to-nearest-even, saturating).
//
// Backward: the block sums dL/ds are binary64 fmas of exact products, added
// in element order 0..15.  Four lanes own one block (4 elements each); the
// running sum walks lane 0 -> 1 -> 2 -> 3 of the quad through DPP moves, so
// the result is the plain sequential sum whatever the launch shape.  Both
// passes are HBM-bound (6.25 / 10.5 bytes per element for tied scales).
#include "common.hpp"
#include "device.hpp"

namespace nvfp4 {

__device__ __forceinline__ float fq_inv(float s) {
  if (s == 0.0f) return 0.0f;
  const float r = 1.0f / s;
  return __builtin_isinf(r) ? __builtin_copysignf(3.40282347e38f, r) : r;
}

// ---------------------------------------------------------------- forward
// A lane owns 4 consecutive elements (one contiguous float4 store per lane);
// 4 lanes share a block's scales.
constexpr int kFqUnroll = 4;

// AMAX: the per-block parameters are amaxes a, the scales s = fl(a / 6), and
// the scale gradients dL/da = dL/ds / 6 (the binary64 sums divided before
// their rounding): the amax reparameterization of scale learning.
template <bool AMAX>
__device__ __forceinline__ float param_scale(float p) {
  if constexpr (AMAX) return p / 6.0f;
  else return p;
}

template <bool AMAX>
__device__ __forceinline__ double param_grad(double g) {
  if constexpr (AMAX) return g / 6.0;
  else return g;
}

template <bool DUAL, bool AMAX>
__global__ void __launch_bounds__(kThreads)
fakequant_fwd_kernel(const uint2* __restrict__ x, int64_t nquads, const float* __restrict__ s_pre,
                     const float* __restrict__ s_post, float4* __restrict__ xq) {
  const int64_t per_iter = (int64_t)gridDim.x * kThreads * kFqUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kFqUnroll; base < nquads; base += per_iter) {
    uint2 w[kFqUnroll];
    float sp[kFqUnroll], so[kFqUnroll];
#pragma unroll
    for (int u = 0; u < kFqUnroll; ++u) {
      const int64_t qd = base + u * kThreads + threadIdx.x;
      const bool ok = qd < nquads;
      w[u] = ok ? ld_nt(x + qd) : make_uint2(0, 0);
      sp[u] = ok ? s_pre[qd >> 2] : 0.0f;
      so[u] = DUAL ? (ok ? s_post[qd >> 2] : 0.0f) : sp[u];
    }
#pragma unroll
    for (int u = 0; u < kFqUnroll; ++u) {
      sp[u] = param_scale<AMAX>(sp[u]);
      so[u] = param_scale<AMAX>(so[u]);
    }
#pragma unroll
    for (int u = 0; u < kFqUnroll; ++u) {
      const int64_t qd = base + u * kThreads + threadIdx.x;
      if (qd >= nquads) continue;
      const float inv = fq_inv(sp[u]);
      uint32_t cw = 0;
      cw = NVFP4_CVT_PK_FP4(cw, bf16_lo(w[u].x) * inv, bf16_hi(w[u].x) * inv, 0);
      cw = NVFP4_CVT_PK_FP4(cw, bf16_lo(w[u].y) * inv, bf16_hi(w[u].y) * inv, 1);
      const f32x2 q01 = NVFP4_DEC_PK_FP4(cw, 0), q23 = NVFP4_DEC_PK_FP4(cw, 1);
      st_nt(make_float4(q01[0] * so[u], q01[1] * so[u], q23[0] * so[u], q23[1] * so[u]), xq + qd);
    }
  }
}

// ---------------------------------------------------------------- backward
// Sequential binary64 sum over the quad: after step k, lane k holds the sum of
// elements 0 .. 4k+3 (lane 0 restarts from 0 every step).
__device__ __forceinline__ double quad_seq_sum(const double (&t)[4], const double (&g)[4],
                                               bool first) {
  double acc = 0.0;
#pragma unroll
  for (int step = 0; step < 4; ++step) {
    double in = shift1_in_quad_f64(acc);
    in = first ? 0.0 : in;
    acc = in;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_fma(g[i], t[i], acc);
  }
  return acc;
}

constexpr int kBwUnroll = 2;

template <bool DUAL, bool AMAX>
__global__ void __launch_bounds__(kThreads)
fakequant_bwd_kernel(const uint2* __restrict__ x, const float4* __restrict__ g, int64_t nquads,
                     const float* __restrict__ s_pre, const float* __restrict__ s_post,
                     float4* __restrict__ dx, float* __restrict__ ds_pre,
                     float* __restrict__ ds_post) {
  const int lane4 = threadIdx.x & 3;
  const int64_t per_iter = (int64_t)gridDim.x * kThreads * kBwUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kBwUnroll; base < nquads; base += per_iter) {
    uint2 xw[kBwUnroll];
    float4 gv[kBwUnroll];
    float sp[kBwUnroll], so[kBwUnroll];
#pragma unroll
    for (int u = 0; u < kBwUnroll; ++u) {
      const int64_t qd = base + u * kThreads + threadIdx.x;  // 4-element group
      const bool ok = qd < nquads;
      xw[u] = ok ? ld_nt(x + qd) : make_uint2(0, 0);
      gv[u] = ok ? ld_nt(g + qd) : make_float4(0.f, 0.f, 0.f, 0.f);
      sp[u] = ok ? s_pre[qd >> 2] : 0.0f;
      so[u] = DUAL ? (ok ? s_post[qd >> 2] : 0.0f) : sp[u];
    }
#pragma unroll
    for (int u = 0; u < kBwUnroll; ++u) {
      sp[u] = param_scale<AMAX>(sp[u]);
      so[u] = param_scale<AMAX>(so[u]);
    }
#pragma unroll
    for (int u = 0; u < kBwUnroll; ++u) {
      const int64_t qd = base + u * kThreads + threadIdx.x;
      const bool ok = qd < nquads;
      const float inv = fq_inv(sp[u]);
      const float xs[4] = {bf16_lo(xw[u].x), bf16_hi(xw[u].x), bf16_lo(xw[u].y), bf16_hi(xw[u].y)};
      const float gs[4] = {gv[u].x, gv[u].y, gv[u].z, gv[u].w};
      float y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = xs[i] * inv;
      uint32_t cw = 0;
      cw = NVFP4_CVT_PK_FP4(cw, y[0], y[1], 0);
      cw = NVFP4_CVT_PK_FP4(cw, y[2], y[3], 1);
      const f32x2 q01 = NVFP4_DEC_PK_FP4(cw, 0), q23 = NVFP4_DEC_PK_FP4(cw, 1);
      const float q[4] = {q01[0], q01[1], q23[0], q23[1]};
      bool in[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) in[i] = y[i] >= -6.0f && y[i] <= 6.0f;
      double gd[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) gd[i] = (double)gs[i];
      float o[4];
      if constexpr (!DUAL) {
        double t[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[i] = in[i] ? gs[i] : 0.0f;
          const float d = in[i] ? q[i] - y[i] : (y[i] < -6.0f ? -6.0f : 6.0f);
          t[i] = (double)d;
        }
        const double s = quad_seq_sum(t, gd, lane4 == 0);
        if (ok && lane4 == 3) ds_pre[qd >> 2] = (float)param_grad<AMAX>(s);
      } else {
        const double ratio = sp[u] == 0.0f ? 0.0 : (double)so[u] / (double)sp[u];
        double tq[4], tx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[i] = in[i] ? (float)(gd[i] * ratio) : 0.0f;
          tq[i] = (double)q[i];
          tx[i] = in[i] ? (double)xs[i] : 0.0;
        }
        const double spost = quad_seq_sum(tq, gd, lane4 == 0);
        const double tsum = quad_seq_sum(tx, gd, lane4 == 0);
        if (ok && lane4 == 3) {
          ds_post[qd >> 2] = (float)param_grad<AMAX>(spost);
          const double spd = (double)sp[u];
          ds_pre[qd >> 2] =
              sp[u] == 0.0f ? 0.0f : (float)param_grad<AMAX>(-((double)so[u] * tsum) / (spd * spd));
        }
      }
      if (ok) st_nt(make_float4(o[0], o[1], o[2], o[3]), dx + qd);
    }
  }
}

static int64_t grid_for(int64_t units, int64_t per_wg) {
  int64_t grid = (units + per_wg - 1) / per_wg;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  grid = grid < cap ? grid : cap;
  return grid < 1 ? 1 : grid;
}

template <bool AMAX>
static hipError_t launch_fwd(const FakeQuantArgs& a, hipStream_t s) {
  const int64_t nquads = a.rows * a.cols / 4;
  const int64_t grid = grid_for(nquads, (int64_t)kThreads * kFqUnroll);
  if (a.s_post)
    hipLaunchKernelGGL((fakequant_fwd_kernel<true, AMAX>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                       reinterpret_cast<const uint2*>(a.x), nquads, a.s_pre, a.s_post,
                       reinterpret_cast<float4*>(a.xq));
  else
    hipLaunchKernelGGL((fakequant_fwd_kernel<false, AMAX>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                       reinterpret_cast<const uint2*>(a.x), nquads, a.s_pre, a.s_post,
                       reinterpret_cast<float4*>(a.xq));
  return hipGetLastError();
}

template <bool AMAX>
static hipError_t launch_bwd(const FakeQuantArgs& a, hipStream_t s) {
  const int64_t nquads = a.rows * a.cols / 4;
  const int64_t grid = grid_for(nquads, (int64_t)kThreads * kBwUnroll);
  if (a.s_post)
    hipLaunchKernelGGL((fakequant_bwd_kernel<true, AMAX>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                       reinterpret_cast<const uint2*>(a.x), reinterpret_cast<const float4*>(a.g),
                       nquads, a.s_pre, a.s_post, reinterpret_cast<float4*>(a.dx), a.ds_pre,
                       a.ds_post);
  else
    hipLaunchKernelGGL((fakequant_bwd_kernel<false, AMAX>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                       reinterpret_cast<const uint2*>(a.x), reinterpret_cast<const float4*>(a.g),
                       nquads, a.s_pre, a.s_post, reinterpret_cast<float4*>(a.dx), a.ds_pre,
                       a.ds_post);
  return hipGetLastError();
}

hipError_t launch_fakequant_fwd(const FakeQuantArgs& a, hipStream_t s) {
  return a.amax_param ? launch_fwd<true>(a, s) : launch_fwd<false>(a, s);
}

hipError_t launch_fakequant_bwd(const FakeQuantArgs& a, hipStream_t s) {
  return a.amax_param ? launch_bwd<true>(a, s) : launch_bwd<false>(a, s);
}

}  // namespace nvfp4
