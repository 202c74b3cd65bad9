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
#include "grid_reduce.hpp"
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
// A NaN or an infinity in the block: scale 0xFF, elements 0.  `at(i)` gives
// value i (it is called twice per value: for the amax and the conversion).
template <typename At>
__device__ __forceinline__ uint32_t mxfp8_block(At at, uint32_t hbase, uint32_t (&w)[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; i += 4)
    amax = __builtin_elementwise_maximum(amax, __builtin_elementwise_maximum(
        max3_abs(at(i), at(i + 1), at(i + 2)), __builtin_fabsf(at(i + 3))));
  const bool bad = !(amax <= 3.40282347e38f);  // NaN or infinity
  const uint32_t biased = __float_as_uint(amax) >> 23;
  const uint32_t sb = biased > 8u ? biased - 8u : 0u;  // e + 127
  const float inv = __uint_as_float((254u - (sb & 0xFFu)) << 23);  // 2^-e
  const uint32_t tt = hbase ^ (hbase >> 16);  // shared first step of fmix32
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t v = e4m3_sr_pack4(at(4 * j) * inv, at(4 * j + 1) * inv, at(4 * j + 2) * inv,
                                     at(4 * j + 3) * inv, fmix32_tail(tt ^ (uint32_t)(4 * j)),
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
constexpr int kRqPitch = kSW * 4;  // binary32 tile row pitch (bytes)

// Byte offset, within a tile row, of column c (0 <= c < kSW).  The 16-byte
// piece h of row block b (columns 16b + 4h .. +4) sits at piece slot
// h ^ ((b >> 1) & 3): the eight lanes of one tile row that store their row
// blocks in the same instruction then cover all 32 banks of a 128-byte LDS
// pass instead of four of them; a column read (one row, consecutive columns)
// still touches each bank once per pass.
__host__ __device__ constexpr int rq_col_off(int c) {
  return (c >> 4) * 64 + 16 * (((c >> 2) & 3) ^ ((c >> 5) & 3)) + 4 * (c & 3);
}
// MXFP8 scale bytes are staged for 8 tiles of 64 rows (16 bytes per column).
// Staging them for 32 tiles (64-byte pieces) took 8.7 KiB of LDS, which held
// the walk to 3 workgroups per CU; at 16 bytes 4 fit (33.5 -> 28.7 us at
// 8192x4096, outputs identical), and the scale bytes are 1/32 of the output.
constexpr int kMxStTiles = 8;
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
  float al[kN];  // per-tensor: unused; per row: the row's amax
};

// The loads are unconditional (addresses clamped into the tensor; a block
// outside it is zeroed where it is used): the number of loads in flight is
// then the same on every path, so waiting for the oldest buffer never has to
// wait for the newer ones too.
template <int TARGET, bool ROWSC>
__device__ __forceinline__ void rq_load(RqLoad<TARGET>& L, const uint8_t* __restrict__ codes,
                                        const uint8_t* __restrict__ scales,
                                        const float* __restrict__ row_amax, int64_t rows,
                                        int64_t cols, int64_t r0, int64_t c0) {
#pragma unroll
  for (int u = 0; u < RqLoad<TARGET>::kN; ++u) {
    const int k = u * kThreads + (int)threadIdx.x;
    int64_t r = r0 + (k >> 3), c = c0 + (k & 7) * 16;
    r = r < rows ? r : rows - 1;
    c = c < cols ? c : cols - 16;
    L.cw[u] = ld_nt(reinterpret_cast<const uint2*>(codes + r * (cols >> 1) + (c >> 1)));
    L.sb[u] = (uint32_t)scales[r * (cols >> 4) + (c >> 4)];
    if constexpr (ROWSC) L.al[u] = row_amax[r];
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
  const int64_t tiles_r = (rows + kTR - 1) / kTR, tiles_c = (cols + kSW - 1) / kSW;
  const int64_t units = ((tiles_r + seg - 1) / seg) * tiles_c;
  const int64_t G = gridDim.x, b = blockIdx.x;
  const int64_t v = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;  // XCD b % 8 takes a run
  const int lane = threadIdx.x;
  // this lane's column block.  MXFP8: lanes 2k and 2k + 1 take the two
  // 32-row halves of one tile column, so the two 32-byte halves of each
  // 64-byte output piece leave in one store instruction (8192x4096: 28.92 ->
  // 27.33 us against the halves from lanes 128 apart, i.e. from different
  // wavefronts; the pair's reads of one column meet in a bank, 2-way, and
  // moving the tile's second half by 128 bytes to split them gained nothing)
  const int cb_col = NV ? lane & (kSW - 1) : lane >> 1;
  const int cb_row = NV ? (lane / kSW) * kCB : (lane & 1) * kCB;
  const int col_off = rq_col_off(cb_col);
  // MXFP8 target: the first unit's first two tiles are requested before the
  // outer scale is read, so their latency overlaps that start-up (30.1 ->
  // 28.9 us at 8192x4096).  The NVFP4 target, which also builds its code
  // table there, ran 1.4% slower that way and keeps the plain order.
  RqLoad<TARGET> A, B, C;
  if (!NV && v < units) {
    const int64_t g = v / tiles_c, c0 = (v - g * tiles_c) * kSW, tr0 = g * seg;
    const int64_t tr1 = tr0 + seg < tiles_r ? tr0 + seg : tiles_r;
    rq_load<TARGET, ROWSC>(A, codes, scales, row_amax, rows, cols, tr0 * kTR, c0);
    rq_load<TARGET, ROWSC>(B, codes, scales, row_amax, rows, cols,
                           (tr0 + 1 < tr1 ? tr0 + 1 : tr1 - 1) * kTR, c0);
  }
  TensorScale ts{};
  if constexpr (NV) {
    ts = tensor_scale(*dst_amax, dst_sg);
    build_table<DST_FMT>(tab, ts.alpha);
  }
  const float alpha0 = ROWSC ? 0.0f : outer_alpha(*amax, sg);
  __syncthreads();
  for (int64_t unit = v; unit < units; unit += G) {
    const int64_t g = unit / tiles_c;
    const int64_t c0 = (unit - g * tiles_c) * kSW;
    const int64_t tr0 = g * seg;
    const int64_t tr1 = tr0 + seg < tiles_r ? tr0 + seg : tiles_r;
    int64_t ct_lo = tr0, st_lo = tr0;  // first tile of the open stages
    // Two tiles are in flight ahead of the one being processed.  The three
    // load buffers rotate by name (the walk is unrolled by three): copying a
    // buffer whose loads are outstanding would make the copy wait for them.
    // Past the end of the walk the last tile is requested again (unused).
    auto step = [&](const RqLoad<TARGET>& L, RqLoad<TARGET>& ahead, int64_t tr) {
      const int64_t r0 = tr * kTR;
      const int64_t t_ahead = tr + 2 < tr1 ? tr + 2 : tr1 - 1;
      rq_load<TARGET, ROWSC>(ahead, codes, scales, row_amax, rows, cols, t_ahead * kTR, c0);
      // ---- dequantize the lane's row blocks into the binary32 tile
#pragma unroll
      for (int u = 0; u < RqLoad<TARGET>::kN; ++u) {
        const int k = u * kThreads + lane;
        const bool ok = r0 + (k >> 3) < rows && c0 + (k & 7) * 16 < cols;
        const uint32_t wx = ok ? L.cw[u].x : 0u, wy = ok ? L.cw[u].y : 0u;
        const float D = ok ? decode_scale(SRC_FMT, L.sb[u]) : 0.0f;
        const float a = !ok ? 0.0f : ROWSC ? outer_alpha(L.al[u], sg) : alpha0;
        float4* dst = reinterpret_cast<float4*>(tile + (k >> 3) * kRqPitch + (k & 7) * 64);
        const int sw = ((k & 7) >> 1) & 3;  // piece h goes to slot h ^ sw
        dst[0 ^ sw] = dequant4(NVFP4_DEC_PK_FP4(wx, 0), NVFP4_DEC_PK_FP4(wx, 1), D, a);
        dst[1 ^ sw] = dequant4(NVFP4_DEC_PK_FP4(wx, 2), NVFP4_DEC_PK_FP4(wx, 3), D, a);
        dst[2 ^ sw] = dequant4(NVFP4_DEC_PK_FP4(wy, 0), NVFP4_DEC_PK_FP4(wy, 1), D, a);
        dst[3 ^ sw] = dequant4(NVFP4_DEC_PK_FP4(wy, 2), NVFP4_DEC_PK_FP4(wy, 3), D, a);
      }
      lds_sync();
      // ---- the lane's column block, quantized
      const int64_t c = c0 + cb_col, r = r0 + cb_row;
      const uint64_t idx0 = (uint64_t)c * (uint64_t)rows + (uint64_t)r;  // index in X^T
      const uint32_t hb = hash_base<ROUND_SR, WIDE>(seed, idx0, key0);
      if constexpr (NV) {
        float xc[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          xc[i] = *reinterpret_cast<const float*>(tile + (cb_row + i) * kRqPitch + col_off);
        const BlockOut o = quantize_block_x<DST_FMT, SELECT_6, ROUND_SR>(xc, tab, ts, hb);
        const int wd = (int)(tr % kCtTiles) * (kTR / 8) + (cb_row >> 3);
        ct[cb_col * kCtPitch + wd] = o.c0;
        ct[cb_col * kCtPitch + wd + 1] = o.c1;
        st[cb_col * kStPitch + (int)(tr % kStTiles) * (kTR / 16) + (cb_row >> 4)] = (uint8_t)o.scale;
      } else {
        // all 32 values read at once (occupancy is bounded by LDS, not VGPRs)
        const uint8_t* colp = tile + cb_row * kRqPitch + col_off;
        float xc[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) xc[i] = *reinterpret_cast<const float*>(colp + i * kRqPitch);
        uint32_t w[8];
        const uint32_t sc = mxfp8_block([&xc](int i) { return xc[i]; }, hb, w);
        if (c < cols && r < rows) {  // rows % 32 == 0: a block is whole or absent
          uint4* p = reinterpret_cast<uint4*>(out_t + c * rows + r);
          p[0] = make_uint4(w[0], w[1], w[2], w[3]);
          p[1] = make_uint4(w[4], w[5], w[6], w[7]);
        }
        st[cb_col * kMxStPitch + (int)(tr % kMxStTiles) * 2 + (cb_row >> 5)] = (uint8_t)sc;
      }
      lds_sync();  // staged outputs complete; the tile may be rewritten
      // ---- flush closed stages
      const bool last = tr + 1 == tr1;
      if constexpr (NV) {
        if (last || (tr + 1) % kCtTiles == 0) {
          flush_codes_t<true>(ct, out_t, rows, cols, c0, ct_lo, tr + 1);
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
    };
    if (NV || unit != v) {  // MXFP8: the first unit's tiles were requested above
      rq_load<TARGET, ROWSC>(A, codes, scales, row_amax, rows, cols, tr0 * kTR, c0);
      rq_load<TARGET, ROWSC>(B, codes, scales, row_amax, rows, cols,
                             (tr0 + 1 < tr1 ? tr0 + 1 : tr1 - 1) * kTR, c0);
    }
    int64_t tr = tr0;
    for (; tr + 3 <= tr1; tr += 3) {
      step(A, C, tr);
      step(B, A, tr + 1);
      step(C, B, tr + 2);
    }
    if (tr < tr1) step(A, C, tr);
    if (tr + 1 < tr1) step(B, A, tr + 1);
  }
}

// ---------------------------------------------------------------- dequantized amax
// max |x_hat| over an NVFP4 tensor.  |x_hat| = fl(fl(|q| |D|) alpha) is
// monotone in |q| |D| (q |D| is exact, and multiplying by alpha >= 0 and
// rounding are monotone), so the maximum is fl(max(|q| |D|) alpha): per
// block the largest magnitude code times |D|, the maximum over the tensor
// (or over a row, for per-row alpha_r), one multiply by alpha at the end.
// Maxima are integer maxima of the sign-cleared binary32 patterns (NaN
// beats infinity beats every finite value), as for the tensor amax.
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

template <int FMT>
__device__ __forceinline__ uint32_t qd_bits(uint2 w, uint32_t sb) {
  const float q = NVFP4_DEC_PK_FP4(max_mag_code(w), 0)[0];
  return __float_as_uint(q * __builtin_fabsf(decode_scale(FMT, sb))) & 0x7FFFFFFFu;
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

constexpr int kDqaUnroll = 4;
constexpr int kDqaThreads = 1024;

// The grid maximum of the per-lane values m written to *out by the last
// workgroup (grid_reduce.hpp).
__device__ __forceinline__ void dq_amax_flush(uint32_t m, float* out, uint8_t* ws) {
  uint32_t r;
  if (grid_reduce<MaxU32, kDqaThreads>(ws, m, &r)) out[0] = __uint_as_float(r);
}

// Per-tensor alpha: a lane takes two blocks (a 16-byte chunk of codes, two
// scale bytes) per load, four loads in flight, one workgroup per CU.
template <int FMT>
__global__ void __launch_bounds__(kDqaThreads)
dq_amax_kernel(const uint4* __restrict__ codes, const uint16_t* __restrict__ scales, int64_t npairs,
               int64_t nblocks, const float* __restrict__ amax, float sg,
               float* __restrict__ out, uint8_t* __restrict__ ws) {
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kDqaThreads;
  int64_t i = (int64_t)blockIdx.x * kDqaThreads + threadIdx.x;
  for (; i + (kDqaUnroll - 1) * stride < npairs; i += kDqaUnroll * stride) {
    uint4 w[kDqaUnroll];
    uint32_t s2[kDqaUnroll];
#pragma unroll
    for (int u = 0; u < kDqaUnroll; ++u) {
      w[u] = ld_nt(codes + i + u * stride);
      s2[u] = scales[i + u * stride];
    }
#pragma unroll
    for (int u = 0; u < kDqaUnroll; ++u)
      m = umax(m, umax(qd_bits<FMT>(make_uint2(w[u].x, w[u].y), s2[u] & 0xFFu),
                       qd_bits<FMT>(make_uint2(w[u].z, w[u].w), s2[u] >> 8)));
  }
  for (; i < npairs; i += stride) {
    const uint4 w = ld_nt(codes + i);
    const uint32_t s2 = scales[i];
    m = umax(m, umax(qd_bits<FMT>(make_uint2(w.x, w.y), s2 & 0xFFu),
                     qd_bits<FMT>(make_uint2(w.z, w.w), s2 >> 8)));
  }
  if ((nblocks & 1) && blockIdx.x == 0 && threadIdx.x == 0)  // the block after the last pair
    m = umax(m, qd_bits<FMT>(reinterpret_cast<const uint2*>(codes)[nblocks - 1],
                             reinterpret_cast<const uint8_t*>(scales)[nblocks - 1]));
  // an empty tensor (nblocks = 0, amax possibly absent) reduces to 0
  const float alpha = nblocks ? outer_alpha(*amax, sg) : 0.0f;
  dq_amax_flush(__float_as_uint(__uint_as_float(m) * alpha) & 0x7FFFFFFFu, out, ws);
}

// Per-row alpha_r: a wavefront per row (its lanes over the row's blocks,
// four loads in flight), the row maximum times alpha_r.
template <int FMT>
__global__ void __launch_bounds__(kDqaThreads)
dq_amax_rows_kernel(const uint2* __restrict__ codes, const uint8_t* __restrict__ scales,
                    int64_t rows, int64_t row_blocks, const float* __restrict__ row_amax, float sg,
                    float* __restrict__ out, uint8_t* __restrict__ ws) {
  const int l = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * (kDqaThreads / 64);
  uint32_t best = 0;
  for (int64_t r = (int64_t)blockIdx.x * (kDqaThreads / 64) + (threadIdx.x >> 6); r < rows; r += nwaves) {
    const uint2* cr = codes + r * row_blocks;
    const uint8_t* sr = scales + r * row_blocks;
    uint32_t m = 0;
    int64_t j = l;
    for (; j + (kDqaUnroll - 1) * 64 < row_blocks; j += kDqaUnroll * 64) {
      uint2 w[kDqaUnroll];
      uint32_t sb[kDqaUnroll];
#pragma unroll
      for (int u = 0; u < kDqaUnroll; ++u) {
        w[u] = ld_nt(cr + j + u * 64);
        sb[u] = sr[j + u * 64];
      }
#pragma unroll
      for (int u = 0; u < kDqaUnroll; ++u) m = umax(m, qd_bits<FMT>(w[u], sb[u]));
    }
    for (; j < row_blocks; j += 64) m = umax(m, qd_bits<FMT>(ld_nt(cr + j), sr[j]));
    m = wave_reduce<MaxU32>(m);
    const float v = __uint_as_float(m) * outer_alpha(row_amax[r], sg);
    best = umax(best, __float_as_uint(v) & 0x7FFFFFFFu);
  }
  dq_amax_flush(best, out, ws);
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

hipError_t launch_dequantized_amax(const RequantArgs& a, float* out, uint8_t* ws, hipStream_t s) {
  const int64_t nblocks = a.rows * a.cols / 16;
  int64_t cap = (int64_t)device_cu_count();  // one workgroup per CU at most
  cap = cap < kSlots ? cap : kSlots;
  const dim3 bd(kDqaThreads);
  if (a.row_amax != nullptr && nblocks > 0) {
    int64_t grid = (a.rows + kDqaThreads / 64 - 1) / (kDqaThreads / 64);
    grid = grid < cap ? grid : cap;
    const uint2* c = reinterpret_cast<const uint2*>(a.codes);
    if (a.fmt == FMT_UE5M3)
      hipLaunchKernelGGL(dq_amax_rows_kernel<FMT_UE5M3>, dim3((unsigned)grid), bd, 0, s, c, a.scales,
                         a.rows, a.cols / 16, a.row_amax, a.sg, out, ws);
    else
      hipLaunchKernelGGL(dq_amax_rows_kernel<FMT_E4M3>, dim3((unsigned)grid), bd, 0, s, c, a.scales,
                         a.rows, a.cols / 16, a.row_amax, a.sg, out, ws);
    return hipGetLastError();
  }
  // per-tensor alpha, or an empty tensor (one workgroup writes 0)
  const int64_t npairs = nblocks / 2;
  int64_t grid = (npairs + (int64_t)kDqaThreads * kDqaUnroll - 1) / ((int64_t)kDqaThreads * kDqaUnroll);
  grid = grid < cap ? grid : cap;
  grid = grid < 1 ? 1 : grid;
  const uint4* c = reinterpret_cast<const uint4*>(a.codes);
  const uint16_t* sc = reinterpret_cast<const uint16_t*>(a.scales);
  if (a.fmt == FMT_UE5M3)
    hipLaunchKernelGGL(dq_amax_kernel<FMT_UE5M3>, dim3((unsigned)grid), bd, 0, s, c, sc, npairs,
                       nblocks, a.amax, a.sg, out, ws);
  else
    hipLaunchKernelGGL(dq_amax_kernel<FMT_E4M3>, dim3((unsigned)grid), bd, 0, s, c, sc, npairs,
                       nblocks, a.amax, a.sg, out, ws);
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
