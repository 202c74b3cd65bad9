// requant.hip -- re-quantization of NVFP4 tensors for the backward pass on
// gfx950 ("End-to-End 4-Bit Training", "Re-quantization with stochastic
// rounding" and its quantized-linear-layer figure): the forward tensor's
// codes and scales are dequantized to binary32 (q * D * alpha, rounded once),
// transposed, and quantized again along the other dimension with stochastic
// rounding, to NVFP4 (max->6, E2M1 with SR) or to MXFP8 (OCP Microscaling:
// blocks of 32, E8M0 power-of-two scale, E4M3 elements with SR).
//
// Strip walker: a workgroup owns a strip of kSW = 128 source columns and
// walks down it in tiles.  Each lane dequantizes whole source row blocks
// (8 code bytes + 1 scale byte, 16 elements) into a binary32 LDS tile, then
// each lane reads one column block of the tile back (16 rows for NVFP4, 32
// for MXFP8) and quantizes it.  The transposed outputs leave as 64-byte
// pieces per output row: NVFP4 codes and scales and MXFP8 scales through LDS
// staging, MXFP8 elements as the two 32-byte halves of each 64-row tile
// column, written together by the two lanes that own them.
#include "quantize_core.hpp"

namespace nvfp4 {

constexpr int kTargetNvfp4 = 0, kTargetMxfp8 = 1;

// ---------------------------------------------------------------- MXFP8 block
// E4M3 stochastic rounding into byte SEL of `old` (the other bytes are kept):
// gfx950 v_cvt_scalef32_sr_fp8_f32 with unit scale rounds |y| up iff
// (r >> 12) + floor(2^20 p) >= 2^20, p the position of |y| between its two
// E4M3 neighbours; the input must already be clamped to +-448 (above, the
// conversion can round to the NaN code).
template <int SEL>
__device__ __forceinline__ uint32_t sr_fp8_into(uint32_t old, float y, uint32_t r) {
  if constexpr (SEL == 0)
    asm("v_cvt_scalef32_sr_fp8_f32 %0, %1, %2, 1.0" : "+v"(old) : "v"(y), "v"(r));
  else if constexpr (SEL == 1)
    asm("v_cvt_scalef32_sr_fp8_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,0]" : "+v"(old) : "v"(y), "v"(r));
  else if constexpr (SEL == 2)
    asm("v_cvt_scalef32_sr_fp8_f32 %0, %1, %2, 1.0 op_sel:[0,0,0,1]" : "+v"(old) : "v"(y), "v"(r));
  else
    asm("v_cvt_scalef32_sr_fp8_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,1]" : "+v"(old) : "v"(y), "v"(r));
  return old;
}

// Four MXFP8 elements (y already divided by the block scale), clamped to
// +-448 and rounded with their variates h into the four bytes of a word.
__device__ __forceinline__ uint32_t e4m3_sr_pack4(float y0, float y1, float y2, float y3,
                                                  uint32_t h0, uint32_t h1, uint32_t h2, uint32_t h3) {
  uint32_t v = scratch_vgpr();
  v = sr_fp8_into<0>(v, __builtin_amdgcn_fmed3f(y0, -448.0f, 448.0f), h0);
  v = sr_fp8_into<1>(v, __builtin_amdgcn_fmed3f(y1, -448.0f, 448.0f), h1);
  v = sr_fp8_into<2>(v, __builtin_amdgcn_fmed3f(y2, -448.0f, 448.0f), h2);
  v = sr_fp8_into<3>(v, __builtin_amdgcn_fmed3f(y3, -448.0f, 448.0f), h3);
  return v;
}

// One MXFP8 block of 32 values (OCP Microscaling): e = floor(log2 amax) - 8,
// at least -127 (the E8M0 byte is e + 127, read from amax's exponent field);
// elements y = x * 2^-e clamped to +-448, then SR onto E4M3 with the hash of
// element index idx0 + i (hbase = lo32(idx0) ^ key, idx0 a multiple of 32).
// A NaN or an infinity in the block: scale 0xFF, elements 0.
__device__ __forceinline__ uint32_t mxfp8_block(const float (&x)[32], uint32_t hbase,
                                                uint32_t (&w)[8]) {
  float m[11];
#pragma unroll
  for (int j = 0; j < 10; ++j) m[j] = max3_abs(x[3 * j], x[3 * j + 1], x[3 * j + 2]);
  m[10] = __builtin_elementwise_maximum(__builtin_fabsf(x[30]), __builtin_fabsf(x[31]));
  const float m01 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m[0], m[1]), m[2]);
  const float m02 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m[3], m[4]), m[5]);
  const float m03 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m[6], m[7]), m[8]);
  const float m04 = __builtin_elementwise_maximum(m[9], m[10]);
  const float amax = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m01, m02),
                                                   __builtin_elementwise_maximum(m03, m04));
  const bool bad = !(amax <= 3.40282347e38f);  // NaN or infinity
  const uint32_t biased = __float_as_uint(amax) >> 23;
  const uint32_t sb = biased > 8u ? biased - 8u : 0u;  // e + 127
  const float inv = __uint_as_float((254u - (sb & 0xFFu)) << 23);  // 2^-e
  const uint32_t tt = hbase ^ (hbase >> 16);  // shared first step of fmix32
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t v = e4m3_sr_pack4(x[4 * j] * inv, x[4 * j + 1] * inv, x[4 * j + 2] * inv,
                                     x[4 * j + 3] * inv, fmix32_tail(tt ^ (uint32_t)(4 * j)),
                                     fmix32_tail(tt ^ (uint32_t)(4 * j + 1)),
                                     fmix32_tail(tt ^ (uint32_t)(4 * j + 2)),
                                     fmix32_tail(tt ^ (uint32_t)(4 * j + 3)));
    w[j] = bad ? 0u : v;
  }
  return bad ? 0xFFu : sb;
}

// ---------------------------------------------------------------- strip walker
template <int TARGET>
struct RqTile {
  static constexpr int kTR = TARGET == kTargetNvfp4 ? 32 : 64;  // tile height (rows)
  static constexpr int kCB = TARGET == kTargetNvfp4 ? 16 : 32;  // column block (rows)
};
constexpr int kRqPitch = kSW * 4 + 16;  // binary32 tile row pitch (bytes), padded
constexpr int kMxStTiles = 32;          // MXFP8 scales: 32 tiles of 64 rows = 64 bytes
constexpr int kMxStBytes = kMxStTiles * 2;
constexpr int kMxStPitch = kMxStBytes + 4;

// Staged MXFP8 scale bytes of tiles [t_lo, t_hi) of the strip at c0 (one
// byte per 32 rows; consecutive lanes write consecutive bytes of a row of
// the transposed scales).
__device__ __forceinline__ void flush_mx_scales_t(const uint8_t* st, uint8_t* __restrict__ scales_t,
                                                  int64_t rows, int64_t cols, int64_t c0,
                                                  int64_t t_lo, int64_t t_hi) {
  const int64_t row0 = (t_lo / kMxStTiles) * kMxStTiles * 64;
  const int b_lo = (int)(t_lo % kMxStTiles) * 2;
  const int64_t b_end = (rows - row0) / 32;
  int b_hi = (int)((t_hi - 1) % kMxStTiles + 1) * 2;
  if (b_end < b_hi) b_hi = (int)b_end;
  const int64_t stride = rows >> 5;
#pragma unroll 1
  for (int u = 0; u < kSW * kMxStBytes / kThreads; ++u) {
    const int j = u * kThreads + threadIdx.x;
    const int col = j / kMxStBytes, b = j % kMxStBytes;
    if (b >= b_lo && b < b_hi && c0 + col < cols)
      scales_t[(c0 + col) * stride + (row0 >> 5) + b] = st[col * kMxStPitch + b];
  }
}

// Source row blocks a lane dequantizes per tile: block k = u * kThreads +
// lane is tile row k / 8, columns (k % 8) * 16 .. +16 of the strip.
template <int TARGET>
struct RqLoad {
  static constexpr int kN = RqTile<TARGET>::kTR * (kSW / 16) / kThreads;  // 1 or 2
  uint2 cw[kN];
  uint32_t sb[kN];
  float al[kN];
};

template <int TARGET, bool ROWSC>
__device__ __forceinline__ void rq_load(RqLoad<TARGET>& L, const uint8_t* __restrict__ codes,
                                        const uint8_t* __restrict__ scales,
                                        const float* __restrict__ row_amax, float sg, float alpha0,
                                        int64_t rows, int64_t cols, int64_t r0, int64_t c0) {
#pragma unroll
  for (int u = 0; u < RqLoad<TARGET>::kN; ++u) {
    const int k = u * kThreads + (int)threadIdx.x;
    const int64_t r = r0 + (k >> 3), c = c0 + (k & 7) * 16;
    const bool ok = r < rows && c < cols;  // cols % 16 == 0: a block is whole or absent
    L.cw[u] = ok ? ld_nt(reinterpret_cast<const uint2*>(codes + r * (cols >> 1) + (c >> 1)))
                 : make_uint2(0, 0);
    L.sb[u] = ok ? (uint32_t)scales[r * (cols >> 4) + (c >> 4)] : 0u;
    if constexpr (ROWSC) L.al[u] = ok ? outer_alpha(row_amax[r], sg) : 0.0f;
    else L.al[u] = ok ? alpha0 : 0.0f;
  }
}

// Four decoded E2M1 values (two bytes) times the block scale and the outer
// scale: (q * D) * alpha, q * D being exact.
__device__ __forceinline__ float4 dequant4(f32x2 q0, f32x2 q1, float D, float a) {
  return make_float4((q0[0] * D) * a, (q0[1] * D) * a, (q1[0] * D) * a, (q1[1] * D) * a);
}

template <int SRC_FMT, bool ROWSC, int TARGET, int DST_FMT, bool WIDE>
__global__ void __launch_bounds__(kThreads)
requant_t_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                 int64_t rows, int64_t cols, const float* __restrict__ amax,
                 const float* __restrict__ row_amax, float sg, const float* __restrict__ dst_amax,
                 float dst_sg, uint64_t seed, uint32_t key0, uint8_t* __restrict__ out_t,
                 uint8_t* __restrict__ out_scales_t, int64_t seg) {
  constexpr int kTR = RqTile<TARGET>::kTR, kCB = RqTile<TARGET>::kCB;
  constexpr bool NV = TARGET == kTargetNvfp4;
  static_assert(kSW * kTR / kCB == kThreads, "one column block per lane and tile");
  __shared__ f32x2 tab[NV ? FmtTraits<DST_FMT>::kCodes : 1];
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTR * kRqPitch];
  __shared__ uint32_t ct[NV ? kSW * kCtPitch : 1];
  __shared__ uint8_t st[NV ? kSW * kStPitch : kSW * kMxStPitch];
  TensorScale ts{};
  if constexpr (NV) {
    ts = tensor_scale(*dst_amax, dst_sg);
    build_table<DST_FMT>(tab, ts.alpha);
  }
  const float alpha0 = ROWSC ? 0.0f : outer_alpha(*amax, sg);
  __syncthreads();
  const int64_t tiles_r = (rows + kTR - 1) / kTR, tiles_c = (cols + kSW - 1) / kSW;
  const int64_t units = ((tiles_r + seg - 1) / seg) * tiles_c;
  const int64_t G = gridDim.x, b = blockIdx.x;
  const int64_t v = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;  // XCD b % 8 takes a run
  const int lane = threadIdx.x;
  const int cb_col = lane & (kSW - 1), cb_row = (lane / kSW) * kCB;  // this lane's column block
  for (int64_t unit = v; unit < units; unit += G) {
    const int64_t g = unit / tiles_c;
    const int64_t c0 = (unit - g * tiles_c) * kSW;
    const int64_t tr0 = g * seg;
    const int64_t tr1 = tr0 + seg < tiles_r ? tr0 + seg : tiles_r;
    int64_t ct_lo = tr0, st_lo = tr0;  // first tile of the open stages
    RqLoad<TARGET> L;
    rq_load<TARGET, ROWSC>(L, codes, scales, row_amax, sg, alpha0, rows, cols, tr0 * kTR, c0);
    for (int64_t tr = tr0; tr < tr1; ++tr) {
      const int64_t r0 = tr * kTR;
      RqLoad<TARGET> Ln;  // the next tile is requested before this one is processed
      if (tr + 1 < tr1)
        rq_load<TARGET, ROWSC>(Ln, codes, scales, row_amax, sg, alpha0, rows, cols, r0 + kTR, c0);
      // ---- dequantize the lane's row blocks into the binary32 tile
#pragma unroll
      for (int u = 0; u < RqLoad<TARGET>::kN; ++u) {
        const int k = u * kThreads + lane;
        const float D = decode_scale(SRC_FMT, L.sb[u]);
        const float a = L.al[u];
        float4* dst = reinterpret_cast<float4*>(tile + (k >> 3) * kRqPitch + (k & 7) * 64);
        dst[0] = dequant4(NVFP4_DEC_PK_FP4(L.cw[u].x, 0), NVFP4_DEC_PK_FP4(L.cw[u].x, 1), D, a);
        dst[1] = dequant4(NVFP4_DEC_PK_FP4(L.cw[u].x, 2), NVFP4_DEC_PK_FP4(L.cw[u].x, 3), D, a);
        dst[2] = dequant4(NVFP4_DEC_PK_FP4(L.cw[u].y, 0), NVFP4_DEC_PK_FP4(L.cw[u].y, 1), D, a);
        dst[3] = dequant4(NVFP4_DEC_PK_FP4(L.cw[u].y, 2), NVFP4_DEC_PK_FP4(L.cw[u].y, 3), D, a);
      }
      __syncthreads();
      // ---- the lane's column block, quantized
      const int64_t c = c0 + cb_col, r = r0 + cb_row;
      const uint64_t idx0 = (uint64_t)c * (uint64_t)rows + (uint64_t)r;  // index in X^T
      const uint32_t hb = hash_base<ROUND_SR, WIDE>(seed, idx0, key0);
      if constexpr (NV) {
        float xc[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          xc[i] = *reinterpret_cast<const float*>(tile + (cb_row + i) * kRqPitch + cb_col * 4);
        const BlockOut o = quantize_block_x<DST_FMT, SELECT_6, ROUND_SR>(xc, tab, ts, hb);
        const int wd = (int)(tr % kCtTiles) * (kTR / 8) + (cb_row >> 3);
        ct[cb_col * kCtPitch + wd] = o.c0;
        ct[cb_col * kCtPitch + wd + 1] = o.c1;
        st[cb_col * kStPitch + (int)(tr % kStTiles) * (kTR / 16) + (cb_row >> 4)] = (uint8_t)o.scale;
      } else {
        float xc[32];
#pragma unroll
        for (int i = 0; i < 32; ++i)
          xc[i] = *reinterpret_cast<const float*>(tile + (cb_row + i) * kRqPitch + cb_col * 4);
        uint32_t w[8];
        const uint32_t sc = mxfp8_block(xc, hb, w);
        if (c < cols && r < rows) {  // rows % 32 == 0: a block is whole or absent
          uint4* p = reinterpret_cast<uint4*>(out_t + c * rows + r);
          p[0] = make_uint4(w[0], w[1], w[2], w[3]);
          p[1] = make_uint4(w[4], w[5], w[6], w[7]);
        }
        st[cb_col * kMxStPitch + (int)(tr % kMxStTiles) * 2 + (cb_row >> 5)] = (uint8_t)sc;
      }
      __syncthreads();  // staged outputs complete; the tile may be rewritten
      // ---- flush closed stages
      const bool last = tr + 1 == tr1;
      if constexpr (NV) {
        if (last || (tr + 1) % kCtTiles == 0) {
          flush_codes_t(ct, out_t, rows, cols, c0, ct_lo, tr + 1);
          ct_lo = tr + 1;
        }
        if (last || (tr + 1) % kStTiles == 0) {
          flush_scales_t(st, out_scales_t, rows, cols, c0, st_lo, tr + 1);
          st_lo = tr + 1;
        }
      } else {
        if (last || (tr + 1) % kMxStTiles == 0) {
          flush_mx_scales_t(st, out_scales_t, rows, cols, c0, st_lo, tr + 1);
          st_lo = tr + 1;
        }
      }
      if (tr + 1 < tr1) L = Ln;
    }
  }
}

// ---------------------------------------------------------------- dequantized amax
// max |x_hat| over an NVFP4 tensor: per block the largest magnitude code
// times |D| times alpha (x_hat is monotone in |q|), reduced like the tensor
// amax (integer max of the sign-cleared binary32 patterns: NaN beats
// infinity beats every finite value).  A lane takes one block (8 code bytes
// and its scale byte) per step.
__device__ __forceinline__ uint32_t max_mag_code(uint2 w) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t a = (w.x >> (4 * i)) & 7u, b = (w.y >> (4 * i)) & 7u;
    m = m > a ? m : a;
    m = m > b ? m : b;
  }
  return m;
}

template <int FMT, bool ROWSC>
__global__ void __launch_bounds__(kThreads)
dq_amax_kernel(const uint2* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t nblocks,
               int64_t row_blocks, const float* __restrict__ amax, float sg,
               uint32_t* __restrict__ out) {
  const float alpha0 = ROWSC ? 0.0f : outer_alpha(*amax, sg);
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nblocks; i += stride) {
    const uint2 w = ld_nt(codes + i);
    const uint32_t sb = scales[i];
    const float a = ROWSC ? outer_alpha(amax[i / row_blocks], sg) : alpha0;
    const float q = NVFP4_DEC_PK_FP4(max_mag_code(w), 0)[0];
    const float D = __builtin_fabsf(decode_scale(FMT, sb));
    const uint32_t bits = __float_as_uint((q * D) * a) & 0x7FFFFFFFu;
    m = m > bits ? m : bits;
  }
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)m, off, 64);
    m = m > o ? m : o;
  }
  __shared__ uint32_t red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
    for (int w2 = 1; w2 < kThreads / 64; ++w2) r = r > red[w2] ? r : red[w2];
    // the running maximum only grows: skip the atomic when it already covers r
    const uint32_t cur = __hip_atomic_load(out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (r > cur) atomicMax(out, r);
  }
}

__global__ void __launch_bounds__(64) dq_amax_init_kernel(uint32_t* out) {
  if (threadIdx.x == 0) out[0] = 0u;
}

// ---------------------------------------------------------------- dispatch
template <int SRC_FMT, bool ROWSC, int TARGET, int DST_FMT, bool WIDE>
static hipError_t launch_rq_typed(const RequantArgs& a, hipStream_t s) {
  constexpr auto kern = requant_t_kernel<SRC_FMT, ROWSC, TARGET, DST_FMT, WIDE>;
  constexpr int kTR = RqTile<TARGET>::kTR;
  const uint32_t key0 = sr_key(a.seed, 0u);
  const int64_t tiles_r = (a.rows + kTR - 1) / kTR, tiles_c = (a.cols + kSW - 1) / kSW;
  const int64_t target = (int64_t)device_cu_count() * resident_per_cu<kern>();
  int64_t seg = (tiles_r * tiles_c + target - 1) / target;
  seg = seg < 1 ? 1 : (seg > tiles_r ? tiles_r : seg);
  const int64_t units = ((tiles_r + seg - 1) / seg) * tiles_c;
  const int64_t grid = units < target ? units : target;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), 0, s, a.codes, a.scales, a.rows,
                     a.cols, a.amax, a.row_amax, a.sg, a.dst_amax, a.dst_sg, a.seed, key0, a.out_t,
                     a.out_scales_t, seg);
  return hipGetLastError();
}

template <int SRC_FMT, bool ROWSC>
static hipError_t launch_rq_src(const RequantArgs& a, hipStream_t s) {
  // indices reach past 2^32 only in tensors of more than 2^32 elements
  const bool wide = (uint64_t)a.rows * (uint64_t)a.cols > (1ull << 32);
  if (a.target == kTargetMxfp8)
    return wide ? launch_rq_typed<SRC_FMT, ROWSC, kTargetMxfp8, FMT_E4M3, true>(a, s)
                : launch_rq_typed<SRC_FMT, ROWSC, kTargetMxfp8, FMT_E4M3, false>(a, s);
  if (a.dst_fmt == FMT_UE5M3)
    return wide ? launch_rq_typed<SRC_FMT, ROWSC, kTargetNvfp4, FMT_UE5M3, true>(a, s)
                : launch_rq_typed<SRC_FMT, ROWSC, kTargetNvfp4, FMT_UE5M3, false>(a, s);
  return wide ? launch_rq_typed<SRC_FMT, ROWSC, kTargetNvfp4, FMT_E4M3, true>(a, s)
              : launch_rq_typed<SRC_FMT, ROWSC, kTargetNvfp4, FMT_E4M3, false>(a, s);
}

hipError_t launch_requant_t(const RequantArgs& a, hipStream_t s) {
  const bool rowsc = a.row_amax != nullptr;
  if (a.fmt == FMT_UE5M3)
    return rowsc ? launch_rq_src<FMT_UE5M3, true>(a, s) : launch_rq_src<FMT_UE5M3, false>(a, s);
  return rowsc ? launch_rq_src<FMT_E4M3, true>(a, s) : launch_rq_src<FMT_E4M3, false>(a, s);
}

hipError_t launch_dequantized_amax(const RequantArgs& a, float* out, hipStream_t s) {
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
  hipLaunchKernelGGL(dq_amax_init_kernel, dim3(1), dim3(64), 0, s, o);
  const int64_t nblocks = a.rows * a.cols / 16;
  if (nblocks == 0) return hipGetLastError();
  int64_t grid = (nblocks + kThreads - 1) / kThreads;
  const int64_t cap = (int64_t)device_cu_count() * 2;  // one atomic per workgroup
  grid = grid < cap ? grid : cap;
  const bool rowsc = a.row_amax != nullptr;
  const float* am = rowsc ? a.row_amax : a.amax;
  const uint2* c = reinterpret_cast<const uint2*>(a.codes);
  const int64_t rb = a.cols / 16;
  const dim3 gd((unsigned)grid), bd(kThreads);
  if (a.fmt == FMT_UE5M3) {
    if (rowsc) hipLaunchKernelGGL((dq_amax_kernel<FMT_UE5M3, true>), gd, bd, 0, s, c, a.scales, nblocks, rb, am, a.sg, o);
    else hipLaunchKernelGGL((dq_amax_kernel<FMT_UE5M3, false>), gd, bd, 0, s, c, a.scales, nblocks, rb, am, a.sg, o);
  } else {
    if (rowsc) hipLaunchKernelGGL((dq_amax_kernel<FMT_E4M3, true>), gd, bd, 0, s, c, a.scales, nblocks, rb, am, a.sg, o);
    else hipLaunchKernelGGL((dq_amax_kernel<FMT_E4M3, false>), gd, bd, 0, s, c, a.scales, nblocks, rb, am, a.sg, o);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- test hook
__global__ void test_e4m3_sr_kernel(const float* y, const uint32_t* h, int64_t n, uint8_t* codes) {
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n / 4;
       g += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t w = e4m3_sr_pack4(y[4 * g], y[4 * g + 1], y[4 * g + 2], y[4 * g + 3],
                                     h[4 * g], h[4 * g + 1], h[4 * g + 2], h[4 * g + 3]);
    for (int i = 0; i < 4; ++i) codes[4 * g + i] = (uint8_t)(w >> (8 * i));
  }
}

hipError_t launch_test_e4m3_sr(const float* y, const uint32_t* h, int64_t n, uint8_t* codes,
                               hipStream_t s) {
  int64_t g = (n / 4 + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 16;
  g = g < 1 ? 1 : (g < cap ? g : cap);
  hipLaunchKernelGGL(test_e4m3_sr_kernel, dim3((unsigned)g), dim3(256), 0, s, y, h, n, codes);
  return hipGetLastError();
}

}  // namespace nvfp4
