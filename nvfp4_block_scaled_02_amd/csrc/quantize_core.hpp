// quantize_core.hpp -- per-block NVFP4 quantization building blocks shared by
// the quantize kernels (quantize.hip) and the re-quantization kernels
// (requant.hip): scale-code tables, the one-lane-per-block and lane-pair block
// quantizers (E2M1 RNE or SR, max->6 or Four-Over-Six), block amax, SR hash
// bases, the wavefront LDS bounce and the count flush.
//
// Method ("End-to-End 4-Bit Training", "Low-precision formats on Blackwell";
// "UE5M3" blog, 数学推导; "Four Over Six" summaries, Methodologie / Method).
#pragma once
#include <atomic>

#include "common.hpp"
#include "device.hpp"
#include "grid_reduce.hpp"

namespace nvfp4 {

template <int FMT>
struct FmtTraits;
template <>
struct FmtTraits<FMT_E4M3> {
  static constexpr int kCodes = 127;  // finite non-negative codes 0x00..0x7E
  static constexpr uint32_t kNan = 0x7Fu;
};
template <>
struct FmtTraits<FMT_UE5M3> {
  static constexpr int kCodes = 255;  // 0x00..0xFE
  static constexpr uint32_t kNan = 0xFFu;
};

template <int FMT>
__device__ __forceinline__ void build_table(f32x2* tab, float alpha) {
  for (int c = threadIdx.x; c < FmtTraits<FMT>::kCodes; c += blockDim.x)
    tab[c] = scale_entry(FMT, (uint32_t)c, alpha);
}

struct HalfOut {
  uint32_t codes;  // 8 nibbles, element i in nibble i
  uint32_t scale;  // the block's scale byte (same in both lanes of the pair)
  uint32_t four;   // 1 if the block chose max->4
};

// SSE contribution of this lane's 8 elements for one candidate: two fmaf
// chains over elements 0-3 and 4-7 (each from +0), then their sum.
__device__ __forceinline__ float half_sse(uint32_t packed, const float (&x)[8], float S) {
  float q[8];
  e2m1_unpack8(packed, q);
  float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float d = __builtin_fmaf(-q[i], S, x[i]);
    p0 = __builtin_fmaf(d, d, p0);
  }
#pragma unroll
  for (int i = 4; i < 8; ++i) {
    float d = __builtin_fmaf(-q[i], S, x[i]);
    p1 = __builtin_fmaf(d, d, p1);
  }
  return p0 + p1;
}

// Quantize the lane's half block.  Every lane of the wavefront must call it
// (DPP partner exchange).  Stochastic rounding only: hbase = lo32(idx0) ^ key,
// idx0 being the output-orientation index of element 0 of this half and key
// the counter-hash key of its high word.  idx0 is a multiple of 8, so element
// i's hash input lo32(idx0 + i) ^ key equals hbase ^ i.
template <int FMT, int SELECT, int ROUND>
__device__ __forceinline__ HalfOut quantize_half(uint4 w, const f32x2* tab, const TensorScale& ts,
                                                 uint32_t hbase) {
  const float x[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                      bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
  // block amax: IEEE 754-2019 maximum (v_maximum3_f32, NaN-propagating) of
  // |x| over the lane's 8 elements, then over the lane pair
  float m = __builtin_elementwise_maximum(__builtin_fabsf(x[0]), __builtin_fabsf(x[1]));
#pragma unroll
  for (int i = 2; i < 8; ++i) m = __builtin_elementwise_maximum(m, __builtin_fabsf(x[i]));
  const float a = __builtin_elementwise_maximum(m, xor1_f32(m));
  const bool nan_blk = ts.nan || (a != a);
  HalfOut o;
  if constexpr (SELECT == SELECT_6) {
    const uint32_t c6 = encode_pair(FMT, a * ts.k6, 0.0f) & 0xFFu;
    const f32x2 t = tab[c6];
    if constexpr (ROUND == ROUND_RNE) {
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = x[i] * t[1];
      o.codes = e2m1_rne_pack8(y);
    } else {
      f32x2 yp[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) yp[b] = f32x2{x[2 * b] * t[1], x[2 * b + 1] * t[1]};
      const uint32_t t = hbase ^ (hbase >> 16);  // shared first step of fmix32
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = fmix32_tail(t ^ (uint32_t)i);
      o.codes = e2m1_sr_pack8(yp, h, __float_as_uint(x[0]), __float_as_uint(x[1]));
    }
    o.scale = c6;
    o.four = 0;
  } else {
    const uint32_t cc = encode_pair(FMT, a * ts.k6, a * ts.k4);
    const uint32_t c6 = cc & 0xFFu, c4 = cc >> 8;
    const f32x2 t6 = tab[c6], t4 = tab[c4];
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = x[i] * t6[1];
    const uint32_t w6 = e2m1_rne_pack8(y);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = x[i] * t4[1];
    const uint32_t w4 = e2m1_rne_pack8(y);
    float e6 = half_sse(w6, x, t6[0]);
    float e4 = half_sse(w4, x, t4[0]);
    const float o6 = xor1_f32(e6), o4 = xor1_f32(e4);
    e6 = e6 + o6;  // (P0 + P1) + (P2 + P3): addition commutes bitwise
    e4 = e4 + o4;
    const bool four = e4 < e6;
    o.codes = four ? w4 : w6;
    o.scale = four ? c4 : c6;
    o.four = four ? 1u : 0u;
  }
  if (nan_blk) {
    o.codes = 0;
    o.scale = FmtTraits<FMT>::kNan;
    o.four = 0;
  }
  return o;
}

// ---------------------------------------------------------------- one lane per block
struct BlockOut {
  uint32_t c0, c1;  // codes of elements 0-7 and 8-15, element i in nibble i % 8
  uint32_t scale;
  uint32_t four;
};

// SSE of one candidate over a whole block: four fmaf chains over elements
// 4k..4k+3 (each from +0), summed as (P0 + P1) + (P2 + P3).
__device__ __forceinline__ float block_sse(uint32_t w0, uint32_t w1, const float (&x)[16], float S) {
  float qa[8], qb[8];
  e2m1_unpack8(w0, qa);
  e2m1_unpack8(w1, qb);
  float P[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float p = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * k + i;
      const float d = __builtin_fmaf(-(e < 8 ? qa[e] : qb[e - 8]), S, x[e]);
      p = __builtin_fmaf(d, d, p);
    }
    P[k] = p;
  }
  return (P[0] + P[1]) + (P[2] + P[3]);
}

// Error of one candidate over a whole block by the selection rule, from the
// residuals d_e = fmaf(-q_e, S, x_e): the squared error (block_sse), the
// absolute error (the same 4x4 tree with additions of |d|) or the largest
// |d| (an IEEE maximum, order-free).
template <int SELECT>
__device__ __forceinline__ float block_err(uint32_t w0, uint32_t w1, const float (&x)[16], float S) {
  if constexpr (SELECT == SELECT_4OVER6_MAE || SELECT == SELECT_4OVER6_MAXERR) {
    float qa[8], qb[8];
    e2m1_unpack8(w0, qa);
    e2m1_unpack8(w1, qb);
    float d[16];
#pragma unroll
    for (int e = 0; e < 16; ++e)
      d[e] = __builtin_fabsf(__builtin_fmaf(-(e < 8 ? qa[e] : qb[e - 8]), S, x[e]));
    if constexpr (SELECT == SELECT_4OVER6_MAXERR) {
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; e += 2) m = __builtin_elementwise_maximum(m, __builtin_elementwise_maximum(d[e], d[e + 1]));
      return m;
    } else {
      float P[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) P[k] = ((0.0f + d[4 * k]) + d[4 * k + 1] + d[4 * k + 2]) + d[4 * k + 3];
      return (P[0] + P[1]) + (P[2] + P[3]);
    }
  } else {
    return block_sse(w0, w1, x, S);
  }
}

// Quantize a whole block (chunks a, b) in one lane: no partner exchange and
// no duplicated scale encode, which the lane-pair form pays for.  hbase as
// in quantize_half, for element 0 of the block (idx0 a multiple of 16).
__device__ __forceinline__ float max3_abs(float a, float b, float c) {
  return __builtin_elementwise_maximum(
      __builtin_elementwise_maximum(__builtin_fabsf(a), __builtin_fabsf(b)), __builtin_fabsf(c));
}

// DIRECT: {S_EFF, INV_S} of the chosen codes are computed (decode, product,
// correctly rounded reciprocal: the same formula as the LDS table) instead of
// looked up -- for per-row outer scales, where no table is shared.
template <int FMT, bool DIRECT>
__device__ __forceinline__ f32x2 scale_of(const f32x2* tab, uint32_t code, float alpha) {
  if constexpr (DIRECT) return scale_entry(FMT, code, alpha);
  else return tab[code];
}

template <int FMT, int SELECT, int ROUND, bool DIRECT = false>
__device__ __forceinline__ BlockOut quantize_block_x(const float (&x)[16], const f32x2* tab,
                                                     const TensorScale& ts, uint32_t hbase) {
  // block amax as a depth-3 tree of v_maximum3_f32 (IEEE maximum is
  // associative and commutative, NaN included, so the order is immaterial)
  const float m0 = max3_abs(x[0], x[1], x[2]), m1 = max3_abs(x[3], x[4], x[5]);
  const float m2 = max3_abs(x[6], x[7], x[8]), m3 = max3_abs(x[9], x[10], x[11]);
  const float m4 = max3_abs(x[12], x[13], x[14]);
  const float m = __builtin_elementwise_maximum(
      __builtin_elementwise_maximum(__builtin_elementwise_maximum(m0, m1), m2),
      __builtin_elementwise_maximum(__builtin_elementwise_maximum(m3, m4), __builtin_fabsf(x[15])));
  const bool nan_blk = ts.nan || (m != m);
  BlockOut o;
  if constexpr (SELECT == SELECT_6) {
    const uint32_t c6 = encode_pair(FMT, m * ts.k6, 0.0f) & 0xFFu;
    const f32x2 t = scale_of<FMT, DIRECT>(tab, c6, ts.alpha);
    if constexpr (ROUND == ROUND_RNE) {
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = x[i] * t[1];
      o.c0 = e2m1_rne_pack8(y);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = x[8 + i] * t[1];
      o.c1 = e2m1_rne_pack8(y);
    } else {
      const uint32_t tt = hbase ^ (hbase >> 16);  // shared first step of fmix32
      f32x2 yp[4];
      uint32_t h[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) yp[j] = f32x2{x[2 * j] * t[1], x[2 * j + 1] * t[1]};
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = fmix32_tail(tt ^ (uint32_t)i);
      o.c0 = e2m1_sr_pack8(yp, h, __float_as_uint(x[0]), __float_as_uint(x[1]));
#pragma unroll
      for (int j = 0; j < 4; ++j) yp[j] = f32x2{x[8 + 2 * j] * t[1], x[9 + 2 * j] * t[1]};
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = fmix32_tail(tt ^ (uint32_t)(8 + i));
      o.c1 = e2m1_sr_pack8(yp, h, __float_as_uint(x[8]), __float_as_uint(x[9]));
    }
    o.scale = c6;
    o.four = 0;
  } else if constexpr (SELECT == SELECT_SWEEP) {
    // every finite scale code, ascending; a strictly smaller squared error
    // replaces the best (ties keep the smaller code); round-to-nearest only
    auto enc = [&](uint32_t c, uint32_t& w0, uint32_t& w1) {
      const f32x2 t = scale_of<FMT, DIRECT>(tab, c, ts.alpha);
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = x[i] * t[1];
      w0 = e2m1_rne_pack8(y);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = x[8 + i] * t[1];
      w1 = e2m1_rne_pack8(y);
      return block_sse(w0, w1, x, t[0]);
    };
    uint32_t b0, b1;
    float best = enc(0u, b0, b1);
    uint32_t bc = 0;
#pragma unroll 1
    for (uint32_t c = 1; c < (uint32_t)FmtTraits<FMT>::kCodes; ++c) {
      uint32_t w0, w1;
      const float e = enc(c, w0, w1);
      if (e < best) {
        best = e;
        bc = c;
        b0 = w0;
        b1 = w1;
      }
    }
    o.c0 = b0;
    o.c1 = b1;
    o.scale = bc;
    o.four = 0;
  } else {
    const uint32_t cc = encode_pair(FMT, m * ts.k6, m * ts.k4);
    const uint32_t c6 = cc & 0xFFu, c4 = cc >> 8;
    const f32x2 t6 = scale_of<FMT, DIRECT>(tab, c6, ts.alpha);
    const f32x2 t4 = scale_of<FMT, DIRECT>(tab, c4, ts.alpha);
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = x[i] * t6[1];
    const uint32_t a6 = e2m1_rne_pack8(y);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = x[8 + i] * t6[1];
    const uint32_t b6 = e2m1_rne_pack8(y);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = x[i] * t4[1];
    const uint32_t a4 = e2m1_rne_pack8(y);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = x[8 + i] * t4[1];
    const uint32_t b4 = e2m1_rne_pack8(y);
    const float e6 = block_err<SELECT>(a6, b6, x, t6[0]);
    const float e4 = block_err<SELECT>(a4, b4, x, t4[0]);
    const bool four = e4 < e6;
    o.c0 = four ? a4 : a6;
    o.c1 = four ? b4 : b6;
    o.scale = four ? c4 : c6;
    o.four = four ? 1u : 0u;
  }
  if (nan_blk) {
    o.c0 = 0;
    o.c1 = 0;
    o.scale = FmtTraits<FMT>::kNan;
    o.four = 0;
  }
  return o;
}

// 16-point random Hadamard transform of a block in registers ("Four Over Six"
// notes, Method: applied to both inputs of the weight-gradient GEMM; "End-to-
// End 4-Bit Training", Quantized communications: orthogonal, spreads
// outliers): y = H16 diag(s) x / 4 with s_j = -1 iff bit j of `signs` is set,
// as x_j * (+-0.25) and then the fast Walsh-Hadamard butterfly, stages
// h = 1, 2, 4, 8, (t_i, t_{i+h}) -> (t_i + t_{i+h}, t_i - t_{i+h}).
__device__ __forceinline__ void rht16(float (&t)[16], uint32_t signs) {
#pragma unroll
  for (int j = 0; j < 16; ++j) t[j] *= ((signs >> j) & 1u) ? -0.25f : 0.25f;
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (!(i & h)) {
        const float a = t[i], b = t[i + h];
        t[i] = a + b;
        t[i + h] = a - b;
      }
}

// The inverse: t_j = y_j * 0.25, the same butterfly, then the signs.
__device__ __forceinline__ void irht16(float (&t)[16], uint32_t signs) {
#pragma unroll
  for (int j = 0; j < 16; ++j) t[j] *= 0.25f;
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (!(i & h)) {
        const float a = t[i], b = t[i + h];
        t[i] = a + b;
        t[i + h] = a - b;
      }
#pragma unroll
  for (int j = 0; j < 16; ++j) t[j] = ((signs >> j) & 1u) ? -t[j] : t[j];
}

// The block as two 16-byte bf16 chunks; RHT: transformed first.
template <int FMT, int SELECT, int ROUND, bool DIRECT = false, bool RHT = false>
__device__ __forceinline__ BlockOut quantize_block(uint4 a, uint4 b, const f32x2* tab,
                                                   const TensorScale& ts, uint32_t hbase,
                                                   uint32_t rht_signs = 0) {
  float x[16] = {bf16_lo(a.x), bf16_hi(a.x), bf16_lo(a.y), bf16_hi(a.y),
                 bf16_lo(a.z), bf16_hi(a.z), bf16_lo(a.w), bf16_hi(a.w),
                 bf16_lo(b.x), bf16_hi(b.x), bf16_lo(b.y), bf16_hi(b.y),
                 bf16_lo(b.z), bf16_hi(b.z), bf16_lo(b.w), bf16_hi(b.w)};
  if constexpr (RHT) rht16(x, rht_signs);
  return quantize_block_x<FMT, SELECT, ROUND, DIRECT>(x, tab, ts, hbase);
}

// A block (16 values in one lane) quantized with a given block amax instead
// of its own: 16x16 tile scales, where every row and column block of a tile
// takes the tile's amax.  Max->6, round-to-nearest-even; a NaN amax (a NaN
// in the tile) gives the NaN scale code and codes 0.
template <int FMT>
__device__ __forceinline__ BlockOut quantize_block_amax(const float (&x)[16], const f32x2* tab,
                                                        const TensorScale& ts, float amax_t) {
  BlockOut o;
  const uint32_t c6 = encode_pair(FMT, amax_t * ts.k6, 0.0f) & 0xFFu;
  const f32x2 t = tab[c6];
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = x[i] * t[1];
  o.c0 = e2m1_rne_pack8(y);
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = x[8 + i] * t[1];
  o.c1 = e2m1_rne_pack8(y);
  o.scale = c6;
  o.four = 0;
  if (ts.nan || amax_t != amax_t) {
    o.c0 = 0;
    o.c1 = 0;
    o.scale = FmtTraits<FMT>::kNan;
  }
  return o;
}

// NaN-propagating maximum of |x| over a block (a depth-3 tree of maximum3).
__device__ __forceinline__ float block_absmax(const float (&x)[16]) {
  const float m0 = max3_abs(x[0], x[1], x[2]), m1 = max3_abs(x[3], x[4], x[5]);
  const float m2 = max3_abs(x[6], x[7], x[8]), m3 = max3_abs(x[9], x[10], x[11]);
  const float m4 = max3_abs(x[12], x[13], x[14]);
  return __builtin_elementwise_maximum(
      __builtin_elementwise_maximum(__builtin_elementwise_maximum(m0, m1), m2),
      __builtin_elementwise_maximum(__builtin_elementwise_maximum(m3, m4), __builtin_fabsf(x[15])));
}

__device__ __forceinline__ void unpack16(uint4 a, uint4 b, float (&x)[16]) {
  x[0] = bf16_lo(a.x); x[1] = bf16_hi(a.x); x[2] = bf16_lo(a.y); x[3] = bf16_hi(a.y);
  x[4] = bf16_lo(a.z); x[5] = bf16_hi(a.z); x[6] = bf16_lo(a.w); x[7] = bf16_hi(a.w);
  x[8] = bf16_lo(b.x); x[9] = bf16_hi(b.x); x[10] = bf16_lo(b.y); x[11] = bf16_hi(b.y);
  x[12] = bf16_lo(b.z); x[13] = bf16_hi(b.z); x[14] = bf16_lo(b.w); x[15] = bf16_hi(b.w);
}

// Hash base of the 8 elements from index idx0 (a multiple of 8).  WIDE: the
// tensor has more than 2^32 elements, so the key depends on the high word;
// otherwise every index has high word 0 and key0 serves.
template <int ROUND, bool WIDE>
__device__ __forceinline__ uint32_t hash_base(uint64_t seed, uint64_t idx0, uint32_t key0) {
  if constexpr (ROUND != ROUND_SR) return 0u;
  const uint32_t hi = (uint32_t)(idx0 >> 32);
  const uint32_t key = WIDE ? (hi == 0 ? key0 : sr_key(seed, hi)) : key0;
  return (uint32_t)idx0 ^ key;
}

// Adds the grid's per-lane 4/6 counts to *count4 in the same launch
// (grid_count_add: the count rides on each workgroup's arrival), so a
// counting launch keeps the launch shape of a non-counting one.  Every
// workgroup of the grid must call it.
template <int BLOCK>
__device__ __forceinline__ void flush_count(unsigned long long* count4, uint32_t n4, uint8_t* ws) {
  grid_count_add<BLOCK>(ws, n4, count4);
}

// Writes the wavefront's 128 chunks (lane l: chunks l and 64 + l) to its LDS
// region so that lane l can read chunks 2l and 2l + 1 back.  The fences
// and wave barriers keep the compiler from moving LDS accesses across them
// (the hardware runs one wavefront's LDS operations in order): the previous
// group's reads happen before the region is overwritten, the writes before
// the reads that follow.
__device__ __forceinline__ void bounce_pair(uint4* reg, int l, uint4 a, uint4 b) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  reg[l] = a;
  reg[64 + l] = b;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroups of kThreads lanes of kernel KERN one CU holds at once (its
// register and LDS use), at least 1; looked up once per kernel.
template <auto KERN>
static int resident_per_cu() {
  static std::atomic<int> cached{0};
  int n = cached.load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, KERN, kThreads, 0) != hipSuccess || n < 1)
      n = 1;
    cached.store(n, std::memory_order_relaxed);
  }
  return n;
}

// ---------------------------------------------------------------- column-wise staging
// Column-wise outputs of a strip walker (a workgroup owns a strip of kSW
// columns and walks down it in tiles of kTR rows) are staged in LDS and
// written as 64-byte pieces per column: codes every kCtTiles tiles, scale
// bytes every kStTiles tiles (and at the end of the walk).  Pieces below 64
// bytes, or 32-byte pieces written at different times, cost extra DRAM
// writes and bandwidth on MI355X.
constexpr int kSW = 128;                        // strip width (columns)
constexpr int kTR = 32;                         // tile height (rows)
constexpr int kTilePitch = kSW * 2 + 16;         // LDS row pitch (bytes), padded
constexpr int kCtTiles = 4;                     // codes_t: 4 tiles = 64 bytes per column
constexpr int kCtWords = kCtTiles * kTR / 8;    // 16 code words per column per stage
constexpr int kCtPitch = kCtWords + 1;          // LDS pitch (words), padded
constexpr int kStTiles = 32;                    // scales_t: 32 tiles = 64 bytes per column
constexpr int kStBytes = kStTiles * kTR / 16;   // 64 scale bytes per column per stage
constexpr int kStPitch = kStBytes + 4;          // LDS pitch (bytes), padded

// Writes the staged column-wise bytes of tile rows [t_lo, t_hi) (absolute
// tile indices within one stage) of the strip at c0.  Only rows < rows and
// columns < cols are written.  Consecutive lanes write consecutive words (or
// bytes) of one column, so a wavefront store covers whole 64-byte pieces.
// Each lane keeps one position in the stage (a word or byte of a column) and
// walks the columns in steps of kThreads / kCtWords (or / kStBytes), so an
// address is a per-lane offset plus a wavefront-uniform one.  The passes go
// in batches of eight: eight LDS reads issued back to back, then eight
// stores, so that the reads' latency is paid once per batch rather than once
// per pass (same-box A/B against one read and one store per pass: column SR
// at 16384x8192 82.2 -> 80.0 us, column 4/6 with the transform 27.7 -> 26.1,
// 16x16 tiles both layouts 18.9 -> 18.2, NVFP4 re-quantization 25.3 -> 24.5;
// outputs identical).  The uniform offset of the passes is one running scalar
// (+ columns per pass x row stride each pass), made opaque to the compiler
// where it is used: otherwise it hoists every pass's address out of the walk
// and keeps them all live (twice the registers).  One running offset instead
// of one opaque offset per pass also halves the walkers' scalar-register
// spills (fused SR 48 -> 26, NVFP4 re-quantization 30+ -> 11): same-box,
// column 4/6 with the transform 25.43 -> 24.60 us, NVFP4 re-quantization
// 24.53 -> 23.81, 16x16 tiles both layouts 17.99 -> 17.61, column SR 80.1 ->
// 79.5, fused SR 122.2 -> 121.6.
// NT: non-temporal code stores (measured faster for the re-quantization's
// walk, slower for the quantizer's column-wise walk).
template <bool NT = false>
__device__ __forceinline__ void flush_codes_t(const uint32_t* ct, uint8_t* __restrict__ codes_t,
                                              int64_t rows, int64_t cols, int64_t c0,
                                              int64_t t_lo, int64_t t_hi) {
  constexpr int kStep = kThreads / kCtWords;  // columns per pass (16)
  constexpr int kPasses = kSW / kStep;        // 8: one batch
  const int64_t row0 = (t_lo / kCtTiles) * kCtTiles * kTR;  // stage origin (rows)
  const int w_lo = (int)(t_lo % kCtTiles) * (kTR / 8);
  int64_t w_end = (rows - row0) / 8;  // words (8 rows each) inside the tensor
  int w_hi = (int)((t_hi - 1) % kCtTiles + 1) * (kTR / 8);
  if (w_end < w_hi) w_hi = (int)w_end;
  const int wd = threadIdx.x % kCtWords, cl = threadIdx.x / kCtWords;
  if (wd < w_lo || wd >= w_hi) return;
  const int64_t stride = rows >> 1;
  uint8_t* const base = codes_t + c0 * stride + (row0 >> 1);  // uniform
  const int64_t lane_off = (int64_t)cl * stride + wd * 4;
  const bool whole_strip = c0 + kSW <= cols;
  uint32_t v[kPasses];
#pragma unroll
  for (int u = 0; u < kPasses; ++u) v[u] = ct[(u * kStep + cl) * kCtPitch + wd];
  const int64_t step = (int64_t)kStep * stride;
  int64_t su = 0;
#pragma unroll
  for (int u = 0; u < kPasses; ++u, su += step) {
    asm volatile("" : "+s"(su));
    if (whole_strip || c0 + u * kStep + cl < cols) {
      uint32_t* p = reinterpret_cast<uint32_t*>(base + su + lane_off);
      if constexpr (NT) st_nt(v[u], p);
      else *p = v[u];
    }
  }
}

__device__ __forceinline__ void flush_scales_t(const uint8_t* st, uint8_t* __restrict__ scales_t,
                                               int64_t rows, int64_t cols, int64_t c0,
                                               int64_t t_lo, int64_t t_hi) {
  constexpr int kStep = kThreads / kStBytes;  // columns per pass (4)
  constexpr int kBatch = 8;
  static_assert((kSW / kStep) % kBatch == 0, "whole batches");
  const int64_t row0 = (t_lo / kStTiles) * kStTiles * kTR;
  const int b_lo = (int)(t_lo % kStTiles) * (kTR / 16);
  int64_t b_end = (rows - row0) / 16;
  int b_hi = (int)((t_hi - 1) % kStTiles + 1) * (kTR / 16);
  if (b_end < b_hi) b_hi = (int)b_end;
  const int bt = threadIdx.x % kStBytes, cl = threadIdx.x / kStBytes;
  if (bt < b_lo || bt >= b_hi) return;
  const int64_t stride = rows >> 4;
  uint8_t* const base = scales_t + c0 * stride + (row0 >> 4);  // uniform
  const int64_t lane_off = (int64_t)cl * stride + bt;
  const bool whole_strip = c0 + kSW <= cols;
  const int64_t step = (int64_t)kStep * stride;
  int64_t su = 0;
#pragma unroll 1
  for (int u0 = 0; u0 < kSW / kStep; u0 += kBatch) {
    uint8_t v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = st[((u0 + u) * kStep + cl) * kStPitch + bt];
#pragma unroll
    for (int u = 0; u < kBatch; ++u, su += step) {
      asm volatile("" : "+s"(su));
      if (whole_strip || c0 + (u0 + u) * kStep + cl < cols) base[su + lane_off] = v[u];
    }
  }
}

}  // namespace nvfp4
