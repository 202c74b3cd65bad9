// quantize.hip -- NVFP4 block-scaled quantization of bf16 tensors on gfx950.
//
// Method ("End-to-End 4-Bit Training", "Low-precision formats on Blackwell";
// "UE5M3" blog, 数学推导; "Four Over Six" summaries, Methodologie / Method):
// per 16-element block, scale = amax_b / Q under the binary32 outer scale
// alpha, encoded to E4M3 or UE5M3; elements rounded onto E2M1; under
// Four-Over-Six both Q = 6 and Q = 4 are encoded and the lower-SSE one kept.
//
// Mapping: a lane owns 8 consecutive elements (one 16-byte bf16 chunk), the
// lane pair (2m, 2m+1) owns one block; the block amax and the two partial
// SSEs meet through one DPP quad_perm move each.  Both candidates, their
// E2M1 codes (v_cvt_scalef32_pk_fp4_f32) and their exact decodes (for the
// SSE) stay in VGPRs.  Per-code {effective scale, reciprocal} tables live in
// LDS, built once per workgroup from the device amax.
//
// Row-wise blocks: a flat grid-stride stream over 16-byte chunks (blocks
// never straddle rows because cols % 16 == 0).  Column-wise blocks (16
// consecutive rows of a column, written as the row-wise layout of X^T): a
// 64x64 tile is read once, optionally quantized row-wise from registers,
// transposed through LDS with a 16-byte-chunk XOR swizzle (conflict-free
// 16-bit writes, 128-bit reads), and quantized again column-wise.
#include "common.hpp"
#include "device.hpp"

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
// (DPP partner exchange).  idx0 = output-orientation index of element 0 of
// this half (stochastic rounding only); key = counter-hash key of its high
// word.
template <int FMT, int SELECT, int ROUND>
__device__ __forceinline__ HalfOut quantize_half(uint4 w, const f32x2* tab, const TensorScale& ts,
                                                 uint32_t key, uint32_t idx0_lo) {
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
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = x[i] * t[1];
    if constexpr (ROUND == ROUND_RNE) {
      o.codes = e2m1_rne_pack8(y);
    } else {
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = fmix32((idx0_lo + i) ^ key);
      o.codes = e2m1_sr_pack8(y, h);
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

__device__ __forceinline__ uint32_t key_for(uint64_t seed, uint64_t idx, uint32_t key0) {
  const uint32_t hi = (uint32_t)(idx >> 32);
  return hi == 0 ? key0 : sr_key(seed, hi);
}

// Adds the per-lane 4/6 counts of the workgroup to *count4 (one atomic).
// Same-address device atomics serialize (about 8 ns each on MI355X), so the
// launchers keep the grid of a counting launch to about one workgroup per CU.
template <int BLOCK>
__device__ __forceinline__ void flush_count(unsigned long long* count4, uint32_t n4) {
  __shared__ uint32_t red[BLOCK / 64];
  for (int off = 32; off >= 1; off >>= 1) n4 += (uint32_t)__shfl_xor((int)n4, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = n4;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long t = 0;
    for (int i = 0; i < BLOCK / 64; ++i) t += red[i];
    if (t) atomicAdd(count4, t);
  }
}

// ---------------------------------------------------------------- row-wise
// Workgroup tile = 256 lanes x kRowUnroll chunks; full tiles run without
// bounds checks, the one partial tile (if any) with them.  Loads are
// non-temporal; code stores (4 bytes per lane) and scale stores (1 byte per
// lane pair) are plain.  The kernel is VALU-bound (about 120 VALU
// instructions per 8 elements for Four-Over-Six), so nothing is spent on
// gathering scale bytes into wider stores.
constexpr int kRowUnroll = 4;

template <int FMT, int SELECT, int ROUND, int BLOCK>
__global__ void __launch_bounds__(BLOCK)
quantize_rows_kernel(const uint4* __restrict__ x, int64_t nchunks, const float* __restrict__ amax,
                     float sg, uint64_t seed, uint32_t key0, uint32_t* __restrict__ codes,
                     uint8_t* __restrict__ scales, unsigned long long* count4) {
  __shared__ f32x2 tab[FmtTraits<FMT>::kCodes];
  const TensorScale ts = tensor_scale(*amax, sg);
  build_table<FMT>(tab, ts.alpha);
  __syncthreads();
  constexpr int64_t kTileChunks = (int64_t)BLOCK * kRowUnroll;
  const bool even = (threadIdx.x & 1) == 0;
  uint32_t n4 = 0;
  const int64_t per_iter = (int64_t)gridDim.x * kTileChunks;
  const int64_t nfull = (nchunks / kTileChunks) * kTileChunks;
  int64_t base = (int64_t)blockIdx.x * kTileChunks;
  for (; base < nfull; base += per_iter) {
    uint4 w[kRowUnroll];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) w[u] = ld_nt(x + base + u * BLOCK + threadIdx.x);
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int64_t ch = base + u * BLOCK + threadIdx.x;
      const uint64_t idx0 = (uint64_t)ch * kChunk;
      const uint32_t key = ROUND == ROUND_SR ? key_for(seed, idx0, key0) : 0u;
      const HalfOut o = quantize_half<FMT, SELECT, ROUND>(w[u], tab, ts, key, (uint32_t)idx0);
      codes[ch] = o.codes;
      if (even) scales[ch >> 1] = (uint8_t)o.scale;
      n4 += even ? o.four : 0u;
    }
  }
  if (base < nchunks) {
    uint4 w[kRowUnroll];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int64_t ch = base + u * BLOCK + threadIdx.x;
      w[u] = ch < nchunks ? ld_nt(x + ch) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int64_t ch = base + u * BLOCK + threadIdx.x;
      const uint64_t idx0 = (uint64_t)ch * kChunk;
      const uint32_t key = ROUND == ROUND_SR ? key_for(seed, idx0, key0) : 0u;
      const HalfOut o = quantize_half<FMT, SELECT, ROUND>(w[u], tab, ts, key, (uint32_t)idx0);
      if (ch < nchunks) {
        codes[ch] = o.codes;
        if (even) scales[ch >> 1] = (uint8_t)o.scale;
        n4 += even ? o.four : 0u;
      }
    }
  }
  if (SELECT == SELECT_4OVER6 && count4) flush_count<BLOCK>(count4, n4);
}

// ---------------------------------------------------------------- column-wise
constexpr int kTile = 64;                  // 64 x 64 bf16 tile
constexpr int kTileChunks = kTile * kTile / kChunk;  // 512 chunks
constexpr int kPerThread = kTileChunks / kThreads;   // 2

// LDS address (in bf16 units) of element (col, row) of the transposed tile:
// column lines of 64 rows, 16-byte row-chunks XOR-swizzled by col / 8.
__device__ __forceinline__ int tpos(int col, int row) {
  return col * kTile + ((((row >> 3) ^ (col >> 3)) & 7) << 3) + (row & 7);
}

template <int FMT, int SELECT, int ROUND, bool DO_ROW>
__global__ void __launch_bounds__(kThreads)
quantize_tiles_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                      const float* __restrict__ amax, float sg, uint64_t seed, uint32_t key0,
                      uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                      uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t,
                      unsigned long long* count4) {
  __shared__ f32x2 tab[FmtTraits<FMT>::kCodes];
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTile * kTile];
  const TensorScale ts = tensor_scale(*amax, sg);
  build_table<FMT>(tab, ts.alpha);
  __syncthreads();
  const bool even = (threadIdx.x & 1) == 0;
  uint32_t n4 = 0;
  const int64_t tiles_r = (rows + kTile - 1) / kTile, tiles_c = (cols + kTile - 1) / kTile;
  const int64_t ntiles = tiles_r * tiles_c;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t r0 = (t / tiles_c) * kTile, c0 = (t % tiles_c) * kTile;
    // ---- load (and optionally quantize row-wise) chunks of 8 columns
    uint4 w[kPerThread];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int k = u * kThreads + threadIdx.x;  // 8 chunks per tile row
      const int64_t r = r0 + (k >> 3), c = c0 + ((k & 7) << 3);
      const bool ok = r < rows && c < cols;
      w[u] = ok ? ld_nt(reinterpret_cast<const uint4*>(x + r * cols + c))
                : make_uint4(0, 0, 0, 0);
    }
    if constexpr (DO_ROW) {
#pragma unroll
      for (int u = 0; u < kPerThread; ++u) {
        const int k = u * kThreads + threadIdx.x;
        const int64_t r = r0 + (k >> 3), c = c0 + ((k & 7) << 3);
        const uint64_t idx0 = (uint64_t)r * (uint64_t)cols + (uint64_t)c;
        const uint32_t key = ROUND == ROUND_SR ? key_for(seed, idx0, key0) : 0u;
        const HalfOut o = quantize_half<FMT, SELECT, ROUND>(w[u], tab, ts, key, (uint32_t)idx0);
        if (r < rows && c < cols) {
          *reinterpret_cast<uint32_t*>(codes + r * (cols >> 1) + (c >> 1)) = o.codes;
          if (even) scales[r * (cols >> 4) + (c >> 4)] = (uint8_t)o.scale;
          n4 += even ? o.four : 0u;
        }
      }
    }
    // ---- transpose through LDS
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int k = u * kThreads + threadIdx.x;
      const int row = k >> 3, col = (k & 7) << 3;
      const uint32_t v[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        tile[tpos(col + j, row)] = (uint16_t)(v[j >> 1] >> ((j & 1) * 16));
    }
    __syncthreads();
    // ---- column-wise: chunk = 8 consecutive rows of one column
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int k = u * kThreads + threadIdx.x;  // 8 chunks per tile column
      const int col = k >> 3, rch = k & 7;
      const uint4 wt = *reinterpret_cast<const uint4*>(tile + tpos(col, rch << 3));
      const int64_t c = c0 + col, r = r0 + (rch << 3);
      const uint64_t idx0 = (uint64_t)c * (uint64_t)rows + (uint64_t)r;
      const uint32_t key = ROUND == ROUND_SR ? key_for(seed, idx0, key0) : 0u;
      const HalfOut o = quantize_half<FMT, SELECT, ROUND>(wt, tab, ts, key, (uint32_t)idx0);
      if (r < rows && c < cols) {
        *reinterpret_cast<uint32_t*>(codes_t + c * (rows >> 1) + (r >> 1)) = o.codes;
        if (even) scales_t[c * (rows >> 4) + (r >> 4)] = (uint8_t)o.scale;
        n4 += even ? o.four : 0u;
      }
    }
    __syncthreads();  // the tile is rewritten by the next iteration
  }
  if (SELECT == SELECT_4OVER6 && count4) flush_count<kThreads>(count4, n4);
}

// ---------------------------------------------------------------- dispatch
template <int FMT, int SELECT, int ROUND>
static hipError_t launch_typed(const QuantizeArgs& a, hipStream_t s) {
  const uint32_t key0 = sr_key(a.seed, 0u);
  const int cus = device_cu_count();
  const bool counting = a.select == SELECT_4OVER6 && a.count4 != nullptr;
  if (a.axes == AXIS_ROW) {
    const int64_t nchunks = a.rows * a.cols / kChunk;
    if (counting) {
      // one 1024-thread workgroup per CU: at most one atomic per CU
      constexpr int B = 1024;
      int64_t grid = (nchunks + (int64_t)B * kRowUnroll - 1) / ((int64_t)B * kRowUnroll);
      grid = grid < cus ? grid : cus;
      hipLaunchKernelGGL((quantize_rows_kernel<FMT, SELECT, ROUND, B>), dim3((unsigned)grid),
                         dim3(B), 0, s, reinterpret_cast<const uint4*>(a.x), nchunks, a.amax,
                         a.sg, a.seed, key0, reinterpret_cast<uint32_t*>(a.codes), a.scales,
                         a.count4);
    } else {
      int64_t grid = (nchunks + (int64_t)kThreads * kRowUnroll - 1) / ((int64_t)kThreads * kRowUnroll);
      const int64_t cap = (int64_t)cus * 8;
      grid = grid < cap ? grid : cap;
      hipLaunchKernelGGL((quantize_rows_kernel<FMT, SELECT, ROUND, kThreads>), dim3((unsigned)grid),
                         dim3(kThreads), 0, s, reinterpret_cast<const uint4*>(a.x), nchunks,
                         a.amax, a.sg, a.seed, key0, reinterpret_cast<uint32_t*>(a.codes),
                         a.scales, a.count4);
    }
    return hipGetLastError();
  }
  const int64_t ntiles = ((a.rows + kTile - 1) / kTile) * ((a.cols + kTile - 1) / kTile);
  const int64_t cap = (int64_t)cus * (counting ? 2 : 8);
  const int64_t grid = ntiles < cap ? ntiles : cap;
  if (a.axes == (AXIS_ROW | AXIS_COL)) {
    hipLaunchKernelGGL((quantize_tiles_kernel<FMT, SELECT, ROUND, true>), dim3((unsigned)grid),
                       dim3(kThreads), 0, s, a.x, a.rows, a.cols, a.amax, a.sg, a.seed, key0,
                       a.codes, a.scales, a.codes_t, a.scales_t, a.count4);
  } else {
    hipLaunchKernelGGL((quantize_tiles_kernel<FMT, SELECT, ROUND, false>), dim3((unsigned)grid),
                       dim3(kThreads), 0, s, a.x, a.rows, a.cols, a.amax, a.sg, a.seed, key0,
                       a.codes, a.scales, a.codes_t, a.scales_t, a.count4);
  }
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_fmt(const QuantizeArgs& a, hipStream_t s) {
  if (a.rounding == ROUND_SR) return launch_typed<FMT, SELECT_6, ROUND_SR>(a, s);
  if (a.select == SELECT_4OVER6) return launch_typed<FMT, SELECT_4OVER6, ROUND_RNE>(a, s);
  return launch_typed<FMT, SELECT_6, ROUND_RNE>(a, s);
}

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t s) {
  if (a.fmt == FMT_E4M3) return launch_fmt<FMT_E4M3>(a, s);
  return launch_fmt<FMT_UE5M3>(a, s);
}

}  // namespace nvfp4
