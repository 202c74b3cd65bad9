// quantize.hip -- NVFP4 block-scaled quantization of bf16 tensors on gfx950.
//
// Method ("End-to-End 4-Bit Training", "Low-precision formats on Blackwell";
// "UE5M3" blog, 数学推导; "Four Over Six" summaries, Methodologie / Method):
// per 16-element block, scale = amax_b / Q under the binary32 outer scale
// alpha, encoded to E4M3 or UE5M3; elements rounded onto E2M1; under
// Four-Over-Six both Q = 6 and Q = 4 are encoded and the lower-SSE one kept.
//
// Two block mappings.  One lane per block (quantize_block): the lane holds
// all 16 elements, both 4/6 candidates, their E2M1 codes
// (v_cvt_scalef32_pk_fp4_f32) and exact decodes (for the SSE) in VGPRs; used
// by every path whose per-block arithmetic dominates (Four-Over-Six,
// stochastic rounding, column-wise).  A lane pair per block (quantize_half):
// 8 elements per lane, block amax and partial SSEs meeting through one DPP
// move each; used by the memory-bound row-wise max->6 round-to-nearest
// stream.  Per-code {effective scale, reciprocal} tables live in LDS, built
// once per workgroup from the device amax.
//
// Row-wise blocks: grid-stride streams over the tensor (blocks never
// straddle rows because cols % 16 == 0).  Column-wise blocks (16 consecutive
// rows of a column, written as the row-wise layout of X^T): a strip walker
// that reads each 32 x 128 tile once into LDS, quantizes it row-wise and/or
// column-wise from there, and stages the column-wise outputs so that they
// leave as 64-byte pieces.
#include "quantize_core.hpp"

namespace nvfp4 {

// ---------------------------------------------------------------- row-wise
// Workgroup tile = 256 lanes x kRowUnroll chunks; full tiles run without
// bounds checks, the one partial tile (if any) with them.  Loads are
// non-temporal; code stores (4 bytes per lane) and scale stores (1 byte per
// lane pair) are plain.  The kernel is VALU-bound (about 120 VALU
// instructions per 8 elements for Four-Over-Six), so nothing is spent on
// gathering scale bytes into wider stores.
constexpr int kRowUnroll = 4;

template <int FMT, int SELECT, int ROUND, bool WIDE, int BLOCK>
__global__ void __launch_bounds__(BLOCK)
quantize_rows_kernel(const uint4* __restrict__ x, int64_t nchunks, const float* __restrict__ amax,
                     float sg, uint64_t seed, uint32_t key0, uint32_t* __restrict__ codes,
                     uint8_t* __restrict__ scales, unsigned long long* count4, uint8_t* ws) {
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
      const uint32_t hb = hash_base<ROUND, WIDE>(seed, (uint64_t)ch * kChunk, key0);
      const HalfOut o = quantize_half<FMT, SELECT, ROUND>(w[u], tab, ts, hb);
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
      const uint32_t hb = hash_base<ROUND, WIDE>(seed, (uint64_t)ch * kChunk, key0);
      const HalfOut o = quantize_half<FMT, SELECT, ROUND>(w[u], tab, ts, hb);
      if (ch < nchunks) {
        codes[ch] = o.codes;
        if (even) scales[ch >> 1] = (uint8_t)o.scale;
        n4 += even ? o.four : 0u;
      }
    }
  }
  if (is_four_six(SELECT) && count4) flush_count<BLOCK>(count4, n4, ws);
}


// Row-wise, one lane per block (Four-Over-Six and stochastic rounding, whose
// per-block work dominates).  A wavefront handles groups of 64 blocks (128
// chunks, 2 KiB): it loads them with two fully coalesced 16-byte loads per
// lane, bounces them through its own 2 KiB of LDS (no workgroup barrier:
// LDS operations of one wavefront complete in order) and each lane reads
// back its two adjacent chunks.  Loading a lane's two chunks directly would
// leave every load instruction half-dense, which costs about 10% of the
// memory rate on the max->6 path.  Codes are stored 8 bytes per lane, scale
// bytes 1 per lane: whole 512- and 64-byte pieces per wavefront.  Register
// use is held to 64 so that 8 wavefronts per SIMD stay resident.
//
// Work distribution: workgroup b owns the groups b*W + j + k*nwaves (W
// wavefronts per workgroup, slot j < W, round k: the grid-stride order), as
// a list of tasks t = k*W + j that its wavefronts take in order from a
// counter in LDS.  Each wavefront starts with task j = its index and takes
// its next task before computing the current one, so its next loads still go
// out right after its stores.  The wavefronts of a SIMD do not progress
// alike (the older ones win the VALU arbitration); with a fixed share each,
// the workgroup waited for its slowest wavefronts (1.7-2.7 us of spread at
// 8192x4096).  Taking tasks as they finish shortened the SR row stream at
// 16384x8192 from 63.0 to 60.0-60.8 us, the scale sweep from 526 to 519 us,
// and the 4/6 quantizer at 8192x4096 from 16.08 to 15.80 us (17.65 to 17.20
// with the count; medians of 21 interleaved runs; outputs identical).  With
// fewer than three groups per wavefront (4096x4096: two) there is little to
// even out and the counter only adds its latency, so each wavefront keeps the
// fixed grid-stride share there (tasks j, j + W, ...).  Across the two
// workgroups of a CU the balance comes from the issue priority
// (ProgressPriority, 1024-lane launches only): it follows the task index, in
// both modes.
template <int FMT, int SELECT, int ROUND, bool WIDE, int BLOCK, bool RHT>
__device__ __forceinline__ void blocks_body(const uint4* __restrict__ x, int64_t nblocks,
                                            const float* __restrict__ amax, float sg, uint64_t seed,
                                            uint32_t key0, uint2* __restrict__ codes,
                                            uint8_t* __restrict__ scales,
                                            unsigned long long* count4, uint8_t* ws,
                                            uint32_t rht_signs) {
  constexpr int W = BLOCK / 64;  // wavefronts per workgroup
  __shared__ f32x2 tab[FmtTraits<FMT>::kCodes];
  __shared__ __attribute__((aligned(16))) uint4 stage[BLOCK * 2];
  __shared__ uint64_t next_task;
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
  uint4* reg = stage + wv * 128;  // this wavefront's 2 KiB
  const int64_t nchunks = nblocks * 2;
  const int64_t nwhole = nblocks / 64;  // groups of 64 blocks
  const int64_t nwaves = (int64_t)gridDim.x * W;
  const int64_t g0 = (int64_t)blockIdx.x * W;
  const bool dynamic = nwhole >= 3 * nwaves;
  // task t of this workgroup -> its group (increasing in t)
  auto group_of = [&](uint64_t t) -> int64_t { return g0 + (int64_t)(t % W) + (int64_t)(t / W) * nwaves; };
  uint64_t t = (uint64_t)__builtin_amdgcn_readfirstlane(wv);  // wave-uniform
  int64_t g = group_of(t);
  // The first group's loads go out before the outer scale is read and the
  // table built, so their latency overlaps that start-up instead of
  // following it (every workgroup of the grid is resident from the start).
  // The loads are unconditional (a wavefront without a whole group reads
  // clamped addresses and ignores the data), and nothing before the loop
  // waits on them: the table takes one entry per lane (BLOCK >= codes).
  static_assert(BLOCK >= FmtTraits<FMT>::kCodes, "one table entry per lane");
  const int64_t c0 = (g < nwhole ? g : 0) * 128 + l;
  uint4 a = ld_nt(x + (c0 < nchunks ? c0 : nchunks - 1));
  uint4 b = ld_nt(x + (c0 + 64 < nchunks ? c0 + 64 : nchunks - 1));
  // two 1024-lane workgroups per CU: issue priority from progress (measured
  // on this launch shape only; with eight 256-lane workgroups per CU the
  // later half of the grid is not the later workgroup of each CU)
  constexpr bool kPrio = BLOCK == 1024;
  const ProgressPriority prio((uint64_t)(nwhole / gridDim.x));
  if (kPrio) prio.set(t);
  const TensorScale ts = tensor_scale(*amax, sg);
  if (threadIdx.x < FmtTraits<FMT>::kCodes)
    tab[threadIdx.x] = scale_entry(FMT, threadIdx.x, ts.alpha);
  if (threadIdx.x == 0) next_task = W;  // tasks 0..W-1: the first groups above
  __syncthreads();
  uint32_t n4 = 0;
  // whole groups, unchecked; the next group's loads are issued after this
  // group's stores (not before its arithmetic: that would cost registers)
  while (g < nwhole) {
    uint64_t tn = 0;
    if (dynamic) {
      if (l == 0) tn = __hip_atomic_fetch_add(&next_task, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      tn = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(tn >> 32)) << 32) |
           __builtin_amdgcn_readfirstlane((uint32_t)tn);
    } else {
      tn = t + W;
    }
    if (kPrio) prio.set(tn);
    bounce_pair(reg, l, a, b);
    const int64_t bk = g * 64 + l;
    const uint32_t hb = hash_base<ROUND, WIDE>(seed, (uint64_t)bk * 16, key0);
    const BlockOut o = quantize_block<FMT, SELECT, ROUND, false, RHT>(reg[2 * l], reg[2 * l + 1],
                                                                      tab, ts, hb, rht_signs);
    st_nt(make_uint2(o.c0, o.c1), codes + bk);
    scales[bk] = (uint8_t)o.scale;
    n4 += o.four;
    t = tn;
    g = group_of(t);
    if (g < nwhole) {
      a = ld_nt(x + g * 128 + l);
      b = ld_nt(x + g * 128 + 64 + l);
    }
  }
  // the partial last group (nblocks % 64 blocks), if this wavefront drew it
  if (g == nwhole && nblocks % 64 != 0) {
    const int64_t c0 = g * 128;
    const uint4 a = c0 + l < nchunks ? ld_nt(x + c0 + l) : make_uint4(0, 0, 0, 0);
    const uint4 b = c0 + 64 + l < nchunks ? ld_nt(x + c0 + 64 + l) : make_uint4(0, 0, 0, 0);
    bounce_pair(reg, l, a, b);
    const int64_t bk = g * 64 + l;
    const uint32_t hb = hash_base<ROUND, WIDE>(seed, (uint64_t)bk * 16, key0);
    const BlockOut o = quantize_block<FMT, SELECT, ROUND, false, RHT>(reg[2 * l], reg[2 * l + 1],
                                                                      tab, ts, hb, rht_signs);
    if (bk < nblocks) {
      st_nt(make_uint2(o.c0, o.c1), codes + bk);
      scales[bk] = (uint8_t)o.scale;
      n4 += o.four;
    }
  }
  if (is_four_six(SELECT) && count4) flush_count<BLOCK>(count4, n4, ws);
}

template <int FMT, int SELECT, int ROUND, bool WIDE, int BLOCK>
__global__ void __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(8)))
quantize_blocks_kernel(const uint4* __restrict__ x, int64_t nblocks, const float* __restrict__ amax,
                       float sg, uint64_t seed, uint32_t key0, uint2* __restrict__ codes,
                       uint8_t* __restrict__ scales, unsigned long long* count4, uint8_t* ws) {
  blocks_body<FMT, SELECT, ROUND, WIDE, BLOCK, false>(x, nblocks, amax, sg, seed, key0, codes,
                                                      scales, count4, ws, 0u);
}

// The same with every block transformed by the 16-point random Hadamard
// transform first.  Its butterfly needs more registers than the 64 that
// eight wavefronts per SIMD allow (the capped build spills); held to 72,
// seven fit (2% faster than the uncapped 76).
template <int FMT, int SELECT, int ROUND, bool WIDE, int BLOCK>
__global__ void __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(7)))
quantize_blocks_rht_kernel(const uint4* __restrict__ x, int64_t nblocks,
                           const float* __restrict__ amax, float sg, uint64_t seed, uint32_t key0,
                           uint2* __restrict__ codes, uint8_t* __restrict__ scales,
                           unsigned long long* count4, uint8_t* ws, uint32_t rht_signs) {
  blocks_body<FMT, SELECT, ROUND, WIDE, BLOCK, true>(x, nblocks, amax, sg, seed, key0, codes,
                                                     scales, count4, ws, rht_signs);
}

// ---------------------------------------------------------------- per-row outer scales
// Row-wise quantization with per-row outer scales ("End-to-End 4-Bit
// Training", Recipe details: per-token outer scales for activations): the
// one-lane-per-block stream of quantize_blocks_kernel, where each lane forms
// its block's row constants (alpha_r, K_6, K_4) and the chosen codes'
// {S_EFF, INV_S} itself.  A per-row LDS table would need two workgroup
// barriers per row, which on this stream cost more than the divisions.
template <int FMT, int SELECT, int ROUND, bool WIDE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8)))
quantize_rowscaled_kernel(const uint4* __restrict__ x, int64_t nblocks, int64_t row_blocks,
                          const float* __restrict__ row_amax, float sg, uint64_t seed,
                          uint32_t key0, uint2* __restrict__ codes, uint8_t* __restrict__ scales,
                          unsigned long long* count4, uint8_t* ws) {
  __shared__ __attribute__((aligned(16))) uint4 stage[kThreads * 2];
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
  uint4* reg = stage + wv * 128;
  const int64_t nchunks = nblocks * 2;
  const int64_t ngroups = (nblocks + 63) / 64;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  const bool narrow = (nblocks >> 32) == 0;
  uint32_t n4 = 0;
  for (int64_t g = (int64_t)blockIdx.x * (kThreads / 64) + wv; g < ngroups; g += nwaves) {
    const int64_t c0 = g * 128;
    const bool whole = c0 + 128 <= nchunks;
    const uint4 a = (whole || c0 + l < nchunks) ? ld_nt(x + c0 + l) : make_uint4(0, 0, 0, 0);
    const uint4 b = (whole || c0 + 64 + l < nchunks) ? ld_nt(x + c0 + 64 + l) : make_uint4(0, 0, 0, 0);
    bounce_pair(reg, l, a, b);
    const int64_t bk = g * 64 + l;
    const bool ok = bk < nblocks;
    const int64_t r = narrow ? (int64_t)((uint32_t)bk / (uint32_t)row_blocks) : bk / row_blocks;
    const TensorScale ts = tensor_scale(ok ? row_amax[r] : 0.0f, sg);
    const uint32_t hb = hash_base<ROUND, WIDE>(seed, (uint64_t)bk * 16, key0);
    const BlockOut o = quantize_block<FMT, SELECT, ROUND, true>(reg[2 * l], reg[2 * l + 1], nullptr, ts, hb);
    if (ok) {
      st_nt(make_uint2(o.c0, o.c1), codes + bk);
      scales[bk] = (uint8_t)o.scale;
      n4 += o.four;
    }
  }
  if (is_four_six(SELECT) && count4) flush_count<kThreads>(count4, n4, ws);
}

// Long rows (at least 64 blocks): a wavefront owns whole rows.  Per row it
// builds its own {S_EFF, INV_S} table in its own LDS (no workgroup barrier:
// only this wavefront reads it, and its LDS operations complete in order),
// then streams the row's 64-block groups exactly as quantize_blocks_kernel
// does.  The table's divisions are paid once per row, not once per block.
template <int FMT, int SELECT, int ROUND, bool WIDE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8)))
quantize_rowwave_kernel(const uint4* __restrict__ x, int64_t rows, int64_t row_blocks,
                        const float* __restrict__ row_amax, float sg, uint64_t seed,
                        uint32_t key0, uint2* __restrict__ codes, uint8_t* __restrict__ scales,
                        unsigned long long* count4, uint8_t* ws) {
  constexpr int kTab = (FmtTraits<FMT>::kCodes + 63) / 64 * 64;
  __shared__ __attribute__((aligned(16))) uint4 stage[kThreads * 2];
  __shared__ f32x2 tabs[kThreads / 64][kTab];
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
  uint4* reg = stage + wv * 128;
  f32x2* tab = tabs[wv];
  const int64_t nch = row_blocks * 2;
  const int64_t ngroups = (row_blocks + 63) / 64, nwhole = row_blocks / 64;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  uint32_t n4 = 0;
  for (int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + wv; r < rows; r += nwaves) {
    const uint4* xr = x + r * nch;
    TensorScale ts = tensor_scale(row_amax[r], sg);
    // the row's constants are uniform over the wavefront: keep them in SGPRs
    ts.alpha = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, ts.alpha)));
    ts.k6 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, ts.k6)));
    ts.k4 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, ts.k4)));
    // the previous row's lookups are done before its table is overwritten
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int c = l; c < kTab; c += 64)
      if (c < FmtTraits<FMT>::kCodes) tab[c] = scale_entry(FMT, (uint32_t)c, ts.alpha);
    const uint4* xg = xr + l;
    const int64_t ob0 = r * row_blocks + l;
    int64_t g = 0;
    for (; g < nwhole; ++g) {
      const uint4 a = ld_nt(xg + g * 128), b = ld_nt(xg + g * 128 + 64);
      bounce_pair(reg, l, a, b);  // also orders the table's writes before its reads
      const int64_t ob = ob0 + g * 64;
      const uint32_t hb = hash_base<ROUND, WIDE>(seed, (uint64_t)ob * 16, key0);
      const BlockOut o = quantize_block<FMT, SELECT, ROUND>(reg[2 * l], reg[2 * l + 1], tab, ts, hb);
      st_nt(make_uint2(o.c0, o.c1), codes + ob);
      scales[ob] = (uint8_t)o.scale;
      n4 += o.four;
    }
    if (g < ngroups) {  // the row's partial last group
      const int64_t c0 = g * 128;
      const uint4 a = c0 + l < nch ? ld_nt(xr + c0 + l) : make_uint4(0, 0, 0, 0);
      const uint4 b = c0 + 64 + l < nch ? ld_nt(xr + c0 + 64 + l) : make_uint4(0, 0, 0, 0);
      bounce_pair(reg, l, a, b);
      const int64_t bk = g * 64 + l;
      const int64_t ob = r * row_blocks + bk;
      const uint32_t hb = hash_base<ROUND, WIDE>(seed, (uint64_t)ob * 16, key0);
      const BlockOut o = quantize_block<FMT, SELECT, ROUND>(reg[2 * l], reg[2 * l + 1], tab, ts, hb);
      if (bk < row_blocks) {
        st_nt(make_uint2(o.c0, o.c1), codes + ob);
        scales[ob] = (uint8_t)o.scale;
        n4 += o.four;
      }
    }
  }
  if (is_four_six(SELECT) && count4) flush_count<kThreads>(count4, n4, ws);
}

// Per-token quantization in one launch (row amax and row-scaled blocks),
// rows of at most kPtChunks 16-byte chunks (4096 columns).  A wavefront owns
// whole rows and reads each once: its lanes load the row (up to eight
// 16-byte chunks each, all in flight together), take its amax (the row amax
// kernel's rules: maxima of the sign-cleared bf16 patterns, so NaN beats
// infinity beats every finite value) while copying it into the wavefront's
// 8 KiB of LDS, write the amax, build the row's {S_EFF, INV_S} table, and
// request the next row into the same registers before quantizing this one's
// 64-block groups from LDS, so the next row's loads overlap this row's
// arithmetic.  LDS (36 KiB per 256-lane workgroup) holds four workgroups per
// CU; only the wavefront itself reads its row and table, and its LDS
// operations complete in order, so no workgroup barrier is needed.
constexpr int kPtChunks = 512;
constexpr int kPtPerLane = kPtChunks / 64;

template <int FMT, int SELECT, int ROUND, bool WIDE>
__global__ void __launch_bounds__(kThreads)
quantize_pertoken_kernel(const uint4* __restrict__ x, int64_t rows, int64_t row_blocks,
                         float* __restrict__ row_amax, float sg, uint64_t seed, uint32_t key0,
                         uint2* __restrict__ codes, uint8_t* __restrict__ scales,
                         unsigned long long* count4, uint8_t* ws) {
  constexpr int kTab = (FmtTraits<FMT>::kCodes + 63) / 64 * 64;
  __shared__ __attribute__((aligned(16))) uint4 rowbuf[kThreads / 64][kPtChunks];
  __shared__ f32x2 tabs[kThreads / 64][kTab];
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
  uint4* buf = rowbuf[wv];
  f32x2* tab = tabs[wv];
  const int64_t nch = row_blocks * 2;  // <= kPtChunks
  const int64_t ngroups = (row_blocks + 63) / 64;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  uint32_t n4 = 0;
  int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + wv;
  uint4 w[kPtPerLane];
  auto load_row = [&](int64_t rr) {
    const uint4* xr = x + rr * nch;
#pragma unroll
    for (int u = 0; u < kPtPerLane; ++u)
      if (l + 64 * u < nch) w[u] = xr[l + 64 * u];
  };
  if (r < rows) load_row(r);
  for (; r < rows; r += nwaves) {
    // the previous row's LDS reads are done before its row and table are
    // overwritten (program order; the fences keep the compiler to it)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < kPtPerLane; ++u)
      if (l + 64 * u < nch) {
        buf[l + 64 * u] = w[u];
        const uint32_t v = chunk_abs_max_bits(w[u]);
        m = m > v ? m : v;
      }
    const float am = __uint_as_float(wave_reduce<MaxU32>(m) << 16);
    if (l == 0) row_amax[r] = am;
    TensorScale ts = tensor_scale(am, sg);
    // the row's constants are uniform over the wavefront: keep them in SGPRs
    ts.alpha = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, ts.alpha)));
    ts.k6 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, ts.k6)));
    ts.k4 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, ts.k4)));
#pragma unroll
    for (int c = l; c < kTab; c += 64)
      if (c < FmtTraits<FMT>::kCodes) tab[c] = scale_entry(FMT, (uint32_t)c, ts.alpha);
    if (r + nwaves < rows) load_row(r + nwaves);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t ob0 = r * row_blocks + l;
    for (int64_t g = 0; g < ngroups; ++g) {
      const int64_t bk = g * 64 + l;  // the lane's block in the row
      const int64_t ob = ob0 + g * 64;
      const uint32_t hb = hash_base<ROUND, WIDE>(seed, (uint64_t)ob * 16, key0);
      const BlockOut o = quantize_block<FMT, SELECT, ROUND>(buf[g * 128 + 2 * l], buf[g * 128 + 2 * l + 1],
                                                            tab, ts, hb);
      if (bk < row_blocks) {  // a partial last group's other lanes read stale chunks
        st_nt(make_uint2(o.c0, o.c1), codes + ob);
        scales[ob] = (uint8_t)o.scale;
        n4 += o.four;
      }
    }
  }
  if (is_four_six(SELECT) && count4) flush_count<kThreads>(count4, n4, ws);
}

// ---------------------------------------------------------------- column-wise
// Strip walker.  A workgroup owns a strip of kSW columns and walks down it in
// tiles of kTR rows.  Each tile is read once (16-byte chunks, 256 bytes per
// row) into LDS, optionally quantized row-wise (64 code bytes per row and
// tile: one full 64-byte piece) and quantized column-wise.  Column-wise outputs are staged in LDS and written as 64-byte
// pieces per column: codes every kCtTiles tiles, scale bytes every kStTiles
// tiles (and at the end of the walk).  Pieces below 64 bytes, or 32-byte
// pieces written at different times, cost extra DRAM writes and bandwidth on
// MI355X; 4-byte pieces per tile, as an unstaged 64-row tile would write for
// its scales, run at a fraction of the write bandwidth.
// Loads the lane's chunks of the tile at rows r0.. of the strip (chunk
// k = u * kThreads + lane: tile row k / 16, columns (k % 16) * 8 ..+8).  The
// loads are unconditional, with addresses clamped into the tensor (cols % 8
// == 0, so a chunk is whole or absent): xu is the lane's chunk column in the
// strip, clamped once per strip; row_off[u] = (tile row of load u) * cols, a
// per-lane constant, is clamped to the tensor's last row by one minimum
// against a wavefront-uniform bound (min(a, b) * cols == min(a * cols, b *
// cols)).  Chunks outside the tensor thus repeat in-tensor chunks; they go
// into LDS like the others.  Zeroing them cost eight VALU moves per load on
// every tile, whole or not (the compiler merged the two store paths into one
// select): without it, same-box, fused SR at 16384x8192 121.7 -> 120.8 us,
// column-block 4/6 with the transform 25.07 -> 24.78, 16x16 tiles 17.54 ->
// 17.41.  The loads are branch-free so that waiting for the oldest tile
// never waits for the newer ones.
constexpr int kLoads = kSW * kTR / kChunk / kThreads;  // 2
constexpr int kLoadRows = kThreads / (kSW / 8);        // tile rows per load (16)

__device__ __forceinline__ bool whole_tile(int64_t rows, int64_t cols, int64_t r0, int64_t c0) {
  return r0 + kTR <= rows && c0 + kSW <= cols;
}

// (last row of the tile inside the tensor - r0) * cols
__device__ __forceinline__ int64_t last_row_off(int64_t rows, int64_t cols, int64_t r0) {
  return (rows - 1 - r0 < kTR - 1 ? rows - 1 - r0 : kTR - 1) * cols;
}

__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ xu,
                                          const int64_t (&row_off)[kLoads], int64_t rows,
                                          int64_t cols, int64_t r0, uint4 (&w)[kLoads]) {
  const int64_t lim = last_row_off(rows, cols, r0);
  const uint16_t* p = xu + r0 * cols;
#pragma unroll
  for (int u = 0; u < kLoads; ++u)
    w[u] = ld_nt(reinterpret_cast<const uint4*>(p + (row_off[u] < lim ? row_off[u] : lim)));
}

// Amax of 16x16 tile t from its 16 row-block values in LDS (NaN-propagating).
__device__ __forceinline__ float tile_amax(const float* am, int t) {
  const float4* p = reinterpret_cast<const float4*>(am + t * 16);
  const float4 a = p[0], b = p[1], c = p[2], d = p[3];
  const float x[16] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w, c.x, c.y, c.z, c.w, d.x, d.y, d.z, d.w};
  return block_absmax(x);
}

// Work unit = one strip (kSW columns) over `seg` consecutive tiles, units
// numbered strip-fastest.  Workgroup b takes units v, v + G, ... (G = grid
// size, sized by the launcher to what the GPU holds at once) with v
// renumbering b so that the G/8 workgroups the dispatcher places on one XCD
// (workgroup b on XCD b mod 8) hold consecutive units: neighbouring strips
// then share their row-wise cache lines inside one XCD's L2.
//
// Per tile: the lanes load it with coalesced 16-byte loads (issued one or two
// tiles ahead, see kAhead) and store it into LDS, row-major with a padded pitch
// (conflict-free 16-byte writes and reads); after a barrier,
// lane b quantizes row block b (tile row b / 8, columns (b % 8) * 16 ..+16)
// from two 16-byte LDS reads, and column block b (tile column b % 128, rows
// (b / 128) * 16 ..+16) from sixteen 16-bit reads; both with the
// one-lane-per-block quantizer.  Every per-tile address and SR index is a
// per-lane constant of the walk (or of the unit) plus a wavefront-uniform
// term, and whole tiles skip the bounds checks a partial tile needs.
//
// TILE2D (16x16 tile scales, max->6, RNE): after the tile is in LDS each
// lane stores its row block's amax in LDS, and after a second barrier every
// row and column block takes the amax of its 16x16 tile (the 16 row-block
// values of that tile), so both passes encode with the tile's scale and the
// column-wise codes are the transpose of the row-wise ones.  DO_COL = false
// skips the column-wise pass (row-wise layout only).
template <int FMT, int SELECT, int ROUND, bool WIDE, bool DO_ROW, bool DO_COL = true,
          bool TILE2D = false, bool RHT = false>
__global__ void __launch_bounds__(kThreads)
quantize_tiles_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                      const float* __restrict__ amax, float sg, uint64_t seed, uint32_t key0,
                      uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                      uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t,
                      unsigned long long* count4, uint8_t* ws, int64_t seg,
                      uint32_t rht_signs = 0) {
  static_assert(kSW * kTR / 16 == kThreads, "one row block and one column block per lane");
  static_assert(kLoads * kLoadRows == kTR, "the loads cover the tile");
  static_assert(!(RHT && (DO_ROW || TILE2D)), "the transform applies to column blocks only here");
  constexpr int kAhead = DO_ROW ? 2 : 1;
  // Two tile buffers for the fused max->6 walks (row and column blocks, RNE
  // or SR, 16x16 tiles too): tile t + 1 goes to the other buffer, so the
  // barrier after a tile's reads is needed only where staged outputs are
  // flushed (one tile in four).  Fused SR at 16384x8192: 122.1 / 122.5 vs
  // 123.1 / 123.3 us; 16x16 tiles, both layouts, at 4096x4096: 17.97 vs
  // 18.08 us (interleaved same-box runs).  The fused Four-Over-Six walks
  // would grow from 122 to 129 VGPRs (4 -> 3 wavefronts per SIMD) and keep
  // one buffer.
  constexpr bool kDbuf = DO_ROW && DO_COL && SELECT == SELECT_6;
  __shared__ f32x2 tab[FmtTraits<FMT>::kCodes];
  __shared__ __attribute__((aligned(16))) uint8_t tile_buf[(kDbuf ? 2 : 1) * kTR * kTilePitch];
  __shared__ uint32_t ct[DO_COL ? kSW * kCtPitch : 1];
  __shared__ uint8_t st[DO_COL ? kSW * kStPitch : 1];
  // TILE2D: row-block amaxes, [16x16 tile t = (row / 16) * 8 + col / 16][row % 16]
  __shared__ __attribute__((aligned(16))) float am[TILE2D ? kThreads : 1];
  const TensorScale ts = tensor_scale(*amax, sg);
  build_table<FMT>(tab, ts.alpha);
  __syncthreads();
  uint32_t n4 = 0;
  const int64_t tiles_r = (rows + kTR - 1) / kTR, tiles_c = (cols + kSW - 1) / kSW;
  const int64_t units = ((tiles_r + seg - 1) / seg) * tiles_c;
  const int64_t G = gridDim.x, b = blockIdx.x;
  const int64_t v = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
  const int lane = threadIdx.x;
  const int rb_row = lane >> 3, rb_col = (lane & 7) * 16;  // row block of this lane
  const int cb_col = lane & (kSW - 1), cb_row = (lane / kSW) * 16;  // column block
  // per-lane constants of the walk: the row offsets of the lane's load
  // chunks, its row block's SR index and output offsets at the tile origin
  int64_t row_off[kLoads];
#pragma unroll
  for (int u = 0; u < kLoads; ++u) row_off[u] = (int64_t)(u * kLoadRows + (lane >> 4)) * cols;
  const uint64_t row_idx_l = (uint64_t)rb_row * (uint64_t)cols + (uint64_t)rb_col;
  const int64_t row_code_l = (int64_t)rb_row * (cols >> 1) + (rb_col >> 1);
  const int64_t row_scale_l = (int64_t)rb_row * (cols >> 4) + (rb_col >> 4);
  for (int64_t unit = v; unit < units; unit += G) {
    const int64_t g = unit / tiles_c;
    const int64_t c0 = (unit - g * tiles_c) * kSW;
    const int64_t tr0 = g * seg;
    const int64_t tr1 = tr0 + seg < tiles_r ? tr0 + seg : tiles_r;
    int64_t ct_lo = tr0, st_lo = tr0;  // first tile of the open stages
    // the lane's column block's SR index at row 0 of the strip, and its load
    // chunk's column, clamped into the tensor
    const uint64_t col_idx_l = (uint64_t)(c0 + cb_col) * (uint64_t)rows + (uint64_t)cb_row;
    const int64_t lc = (lane & 15) * 8;
    const uint16_t* const xu = x + c0 + (lc < cols - 8 - c0 ? lc : cols - 8 - c0);
    // kAhead tiles are in flight ahead of the one being processed: two for
    // the fused walk, one for the column-only walk (whose registers then fit
    // five wavefronts per SIMD instead of four, measured 3.5% faster).  The
    // load buffers rotate by name (the walk is unrolled by kAhead + 1):
    // copying a buffer whose loads are outstanding would make the copy wait
    // for them.  Past the end of the walk the last tile is requested again
    // (unused).
    auto step = [&](const uint4 (&w)[kLoads], uint4 (&ahead)[kLoads], int64_t tr) {
      const int64_t r0 = tr * kTR;
      uint8_t* const tile = tile_buf + (kDbuf ? (int)(tr & 1) * (kTR * kTilePitch) : 0);
      const bool whole = whole_tile(rows, cols, r0, c0);
      load_tile(xu, row_off, rows, cols, (tr + kAhead < tr1 ? tr + kAhead : tr1 - 1) * kTR, ahead);
      // ---- into LDS, row-major.  A partial tile's chunks outside the
      // tensor hold copies of clamped in-tensor chunks: rows % 16 == 0 and
      // cols % 16 == 0 (cols % 8 == 0 column-only), so every 16-element
      // block, and every 16x16 tile, is wholly inside or wholly outside, and
      // the outside ones are neither stored nor counted
#pragma unroll
      for (int u = 0; u < kLoads; ++u) {
        const int k = u * kThreads + lane;
        *reinterpret_cast<uint4*>(tile + (k >> 4) * kTilePitch + (k & 15) * 16) = w[u];
      }
      lds_sync();
      if constexpr (TILE2D) {
        float xr[16];
        unpack16(*reinterpret_cast<const uint4*>(tile + rb_row * kTilePitch + rb_col * 2),
                 *reinterpret_cast<const uint4*>(tile + rb_row * kTilePitch + rb_col * 2 + 16), xr);
        am[((rb_row >> 4) * 8 + (rb_col >> 4)) * 16 + (rb_row & 15)] = block_absmax(xr);
        lds_sync();
      }
      // ---- row-wise block
      if constexpr (DO_ROW) {
        const uint4 wa = *reinterpret_cast<const uint4*>(tile + rb_row * kTilePitch + rb_col * 2);
        const uint4 wb = *reinterpret_cast<const uint4*>(tile + rb_row * kTilePitch + rb_col * 2 + 16);
        BlockOut o;
        if constexpr (TILE2D) {
          float xr[16];
          unpack16(wa, wb, xr);
          o = quantize_block_amax<FMT>(xr, tab, ts, tile_amax(am, (rb_row >> 4) * 8 + (rb_col >> 4)));
        } else {
          const uint32_t hb = hash_base<ROUND, WIDE>(seed, row_idx_l + (uint64_t)(r0 * cols + c0), key0);
          o = quantize_block<FMT, SELECT, ROUND>(wa, wb, tab, ts, hb);
        }
        if (whole || (r0 + rb_row < rows && c0 + rb_col < cols)) {
          st_nt(make_uint2(o.c0, o.c1),
                reinterpret_cast<uint2*>(codes + (r0 * (cols >> 1) + (c0 >> 1)) + row_code_l));
          scales[(r0 * (cols >> 4) + (c0 >> 4)) + row_scale_l] = (uint8_t)o.scale;
          n4 += o.four;
        }
      }
      // ---- column-wise block
      if constexpr (DO_COL) {
        float xc[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          xc[i] = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t*>(
                                      tile + (cb_row + i) * kTilePitch + cb_col * 2) << 16);
        if constexpr (RHT) rht16(xc, rht_signs);
        BlockOut o;
        if constexpr (TILE2D) {
          o = quantize_block_amax<FMT>(xc, tab, ts, tile_amax(am, (cb_row >> 4) * 8 + (cb_col >> 4)));
        } else {
          const uint32_t hb = hash_base<ROUND, WIDE>(seed, col_idx_l + (uint64_t)r0, key0);
          o = quantize_block_x<FMT, SELECT, ROUND>(xc, tab, ts, hb);
        }
        const int wd = (int)(tr % kCtTiles) * (kTR / 8) + (cb_row >> 3);
        ct[cb_col * kCtPitch + wd] = o.c0;
        ct[cb_col * kCtPitch + wd + 1] = o.c1;
        st[cb_col * kStPitch + (int)(tr % kStTiles) * (kTR / 16) + (cb_row >> 4)] = (uint8_t)o.scale;
        if (whole || (r0 + cb_row < rows && c0 + cb_col < cols)) n4 += o.four;
      }
      // ---- flush closed stages
      const bool last = tr + 1 == tr1;
      const bool flush_ct = DO_COL && (last || (tr + 1) % kCtTiles == 0);
      const bool flush_st = DO_COL && (last || (tr + 1) % kStTiles == 0);
      // staged outputs complete before a flush reads them; with one tile
      // buffer, also before the next tile overwrites this one (with two, the
      // next tile goes to the other buffer, and the barrier after its LDS
      // writes orders them after every read of this one)
      if (!kDbuf || flush_ct || flush_st) lds_sync();
      if constexpr (DO_COL) {
        if (flush_ct) {
          flush_codes_t(ct, codes_t, rows, cols, c0, ct_lo, tr + 1);
          ct_lo = tr + 1;
        }
        if (flush_st) {
          flush_scales_t(st, scales_t, rows, cols, c0, st_lo, tr + 1);
          st_lo = tr + 1;
        }
      }
    };
    uint4 A[kLoads], B[kLoads], C[kLoads];
    load_tile(xu, row_off, rows, cols, tr0 * kTR, A);
    int64_t tr = tr0;
    if constexpr (kAhead == 2) {
      load_tile(xu, row_off, rows, cols, (tr0 + 1 < tr1 ? tr0 + 1 : tr1 - 1) * kTR, B);
      for (; tr + 3 <= tr1; tr += 3) {
        step(A, C, tr);
        step(B, A, tr + 1);
        step(C, B, tr + 2);
      }
      if (tr < tr1) step(A, C, tr);
      if (tr + 1 < tr1) step(B, A, tr + 1);
    } else {
      for (; tr + 2 <= tr1; tr += 2) {
        step(A, B, tr);
        step(B, A, tr + 1);
      }
      if (tr < tr1) step(A, B, tr);
    }
  }
  if (is_four_six(SELECT) && count4) flush_count<kThreads>(count4, n4, ws);
}

// ---------------------------------------------------------------- dispatch
// Grids never exceed the workspace's kSlots (a counting launch reduces one
// value per workgroup there); every launch below is far smaller on MI355X.
static int64_t cap_grid(int64_t grid, int64_t cap) {
  grid = grid < cap ? grid : cap;
  grid = grid < kSlots ? grid : kSlots;
  return grid < 1 ? 1 : grid;
}

// Strip-walker launch: as many workgroups as the GPU holds at once, each
// walking a strip over `seg` tiles.
template <auto KERN>
static void walker_shape(const QuantizeArgs& a, int64_t& grid, int64_t& seg) {
  const int64_t tiles_r = (a.rows + kTR - 1) / kTR, tiles_c = (a.cols + kSW - 1) / kSW;
  const int64_t target = (int64_t)device_cu_count() * resident_per_cu<KERN>();
  seg = (tiles_r * tiles_c + target - 1) / target;
  seg = seg < 1 ? 1 : (seg > tiles_r ? tiles_r : seg);
  const int64_t units = ((tiles_r + seg - 1) / seg) * tiles_c;
  grid = cap_grid(units, target);
}

template <int FMT, int SELECT, int ROUND, bool WIDE>
static hipError_t launch_typed(const QuantizeArgs& a, hipStream_t s) {
  const uint32_t key0 = sr_key(a.seed, 0u);
  const int cus = device_cu_count();
  if (a.axes == AXIS_ROW) {
    if constexpr (SELECT != SELECT_6 || ROUND == ROUND_SR) {
      // one lane per block: these paths are bound by per-block arithmetic
      const int64_t nblocks = a.rows * a.cols / 16;
      const int64_t ngroups = (nblocks + 63) / 64;
      if (ngroups >= (int64_t)cus * 32) {
        // enough groups to fill every CU: two 1024-thread workgroups per CU
        // (8 wavefronts per SIMD, as with eight of 256) build a quarter of
        // the tables, 16.57 -> 16.0 us at 8192x4096 (same-box A/B)
        constexpr int B = 1024;
        const int64_t grid = cap_grid((ngroups + B / 64 - 1) / (B / 64), (int64_t)cus * 2);
        hipLaunchKernelGGL((quantize_blocks_kernel<FMT, SELECT, ROUND, WIDE, B>), dim3((unsigned)grid),
                           dim3(B), 0, s, reinterpret_cast<const uint4*>(a.x), nblocks, a.amax, a.sg,
                           a.seed, key0, reinterpret_cast<uint2*>(a.codes), a.scales, a.count4, a.ws);
      } else {
        // small tensors: 256-thread workgroups spread the groups over more CUs
        const int64_t grid = cap_grid((ngroups + kThreads / 64 - 1) / (kThreads / 64), (int64_t)cus * 8);
        hipLaunchKernelGGL((quantize_blocks_kernel<FMT, SELECT, ROUND, WIDE, kThreads>),
                           dim3((unsigned)grid), dim3(kThreads), 0, s,
                           reinterpret_cast<const uint4*>(a.x), nblocks, a.amax, a.sg, a.seed, key0,
                           reinterpret_cast<uint2*>(a.codes), a.scales, a.count4, a.ws);
      }
    } else {
      // max->6 with round-to-nearest: the lane-pair stream (no count output)
      const int64_t nchunks = a.rows * a.cols / kChunk;
      const int64_t grid = cap_grid((nchunks + (int64_t)kThreads * kRowUnroll - 1) / ((int64_t)kThreads * kRowUnroll),
                                    (int64_t)cus * 8);
      hipLaunchKernelGGL((quantize_rows_kernel<FMT, SELECT, ROUND, WIDE, kThreads>),
                         dim3((unsigned)grid), dim3(kThreads), 0, s,
                         reinterpret_cast<const uint4*>(a.x), nchunks, a.amax, a.sg, a.seed, key0,
                         reinterpret_cast<uint32_t*>(a.codes), a.scales, a.count4, a.ws);
    }
    return hipGetLastError();
  }
  constexpr auto kFused = quantize_tiles_kernel<FMT, SELECT, ROUND, WIDE, true>;
  constexpr auto kCol = quantize_tiles_kernel<FMT, SELECT, ROUND, WIDE, false>;
  const bool fused = a.axes == (AXIS_ROW | AXIS_COL);
  int64_t grid, seg;
  if (fused) walker_shape<kFused>(a, grid, seg);
  else walker_shape<kCol>(a, grid, seg);
  hipLaunchKernelGGL(fused ? kFused : kCol, dim3((unsigned)grid), dim3(kThreads), 0, s, a.x, a.rows,
                     a.cols, a.amax, a.sg, a.seed, key0, a.codes, a.scales, a.codes_t, a.scales_t,
                     a.count4, a.ws, seg, 0u);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_fmt(const QuantizeArgs& a, hipStream_t s) {
  if (a.rounding == ROUND_SR) {
    // indices reach past 2^32 only in tensors of more than 2^32 elements
    const bool wide = (uint64_t)a.rows * (uint64_t)a.cols > (1ull << 32);
    return wide ? launch_typed<FMT, SELECT_6, ROUND_SR, true>(a, s)
                : launch_typed<FMT, SELECT_6, ROUND_SR, false>(a, s);
  }
  switch (a.select) {
    case SELECT_4OVER6: return launch_typed<FMT, SELECT_4OVER6, ROUND_RNE, false>(a, s);
    case SELECT_4OVER6_MAE: return launch_typed<FMT, SELECT_4OVER6_MAE, ROUND_RNE, false>(a, s);
    case SELECT_4OVER6_MAXERR: return launch_typed<FMT, SELECT_4OVER6_MAXERR, ROUND_RNE, false>(a, s);
    case SELECT_SWEEP: return launch_typed<FMT, SELECT_SWEEP, ROUND_RNE, false>(a, s);
    default: return launch_typed<FMT, SELECT_6, ROUND_RNE, false>(a, s);
  }
}

template <int FMT, int SELECT, int ROUND, bool WIDE>
static hipError_t launch_rowscaled_rows(const QuantizeArgs& a, uint32_t key0, hipStream_t s) {
  const int64_t cus = device_cu_count();
  const int64_t nblocks = a.rows * a.cols / 16;
  const int64_t row_blocks = a.cols / 16;
  // A wavefront per row when its groups are mostly full (at least 3/4 of
  // the lanes busy), else one lane per block over the flat block stream.
  if (row_blocks % 64 == 0 || row_blocks >= 192) {
    const int64_t grid = cap_grid((a.rows + kThreads / 64 - 1) / (kThreads / 64), cus * 8);
    hipLaunchKernelGGL((quantize_rowwave_kernel<FMT, SELECT, ROUND, WIDE>), dim3((unsigned)grid),
                       dim3(kThreads), 0, s, reinterpret_cast<const uint4*>(a.x), a.rows,
                       row_blocks, a.amax, a.sg, a.seed, key0,
                       reinterpret_cast<uint2*>(a.codes), a.scales, a.count4, a.ws);
    return hipGetLastError();
  }
  const int64_t ngroups = (nblocks + 63) / 64;
  const int64_t grid = cap_grid((ngroups + kThreads / 64 - 1) / (kThreads / 64), cus * 8);
  hipLaunchKernelGGL((quantize_rowscaled_kernel<FMT, SELECT, ROUND, WIDE>), dim3((unsigned)grid),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint4*>(a.x), nblocks,
                     a.cols / 16, a.amax, a.sg, a.seed, key0,
                     reinterpret_cast<uint2*>(a.codes), a.scales, a.count4, a.ws);
  return hipGetLastError();
}

// row_amax_out != nullptr: per-token quantization, the row amaxes computed
// and written there (a.amax not read); one launch for rows of at most
// kPtChunks chunks, else the row amax kernel and then the row-scaled one.
template <int FMT, int SELECT, int ROUND, bool WIDE>
static hipError_t launch_rowscaled_typed(const QuantizeArgs& a, float* row_amax_out, hipStream_t s) {
  const uint32_t key0 = sr_key(a.seed, 0u);
  const int64_t cus = device_cu_count();
  const int64_t row_blocks = a.cols / 16;
  if (row_amax_out && row_blocks * 2 <= kPtChunks) {
    const int64_t grid = cap_grid((a.rows + kThreads / 64 - 1) / (kThreads / 64), cus * 4);
    hipLaunchKernelGGL((quantize_pertoken_kernel<FMT, SELECT, ROUND, WIDE>), dim3((unsigned)grid),
                       dim3(kThreads), 0, s, reinterpret_cast<const uint4*>(a.x), a.rows,
                       row_blocks, row_amax_out, a.sg, a.seed, key0,
                       reinterpret_cast<uint2*>(a.codes), a.scales, a.count4, a.ws);
    return hipGetLastError();
  }
  QuantizeArgs b = a;
  if (row_amax_out) {
    const hipError_t e = launch_row_amax(a.x, a.rows, a.cols, row_amax_out, s);
    if (e != hipSuccess) return e;
    b.amax = row_amax_out;
  }
  return launch_rowscaled_rows<FMT, SELECT, ROUND, WIDE>(b, key0, s);
}

template <int FMT>
static hipError_t launch_rowscaled_fmt(const QuantizeArgs& a, float* row_amax_out, hipStream_t s) {
  if (a.rounding == ROUND_SR) {
    const bool wide = (uint64_t)a.rows * (uint64_t)a.cols > (1ull << 32);
    return wide ? launch_rowscaled_typed<FMT, SELECT_6, ROUND_SR, true>(a, row_amax_out, s)
                : launch_rowscaled_typed<FMT, SELECT_6, ROUND_SR, false>(a, row_amax_out, s);
  }
  switch (a.select) {
    case SELECT_4OVER6: return launch_rowscaled_typed<FMT, SELECT_4OVER6, ROUND_RNE, false>(a, row_amax_out, s);
    case SELECT_4OVER6_MAE: return launch_rowscaled_typed<FMT, SELECT_4OVER6_MAE, ROUND_RNE, false>(a, row_amax_out, s);
    case SELECT_4OVER6_MAXERR: return launch_rowscaled_typed<FMT, SELECT_4OVER6_MAXERR, ROUND_RNE, false>(a, row_amax_out, s);
    case SELECT_SWEEP: return launch_rowscaled_typed<FMT, SELECT_SWEEP, ROUND_RNE, false>(a, row_amax_out, s);
    default: return launch_rowscaled_typed<FMT, SELECT_6, ROUND_RNE, false>(a, row_amax_out, s);
  }
}

hipError_t launch_quantize_rowscaled(const QuantizeArgs& a, hipStream_t s) {
  return a.fmt == FMT_E4M3 ? launch_rowscaled_fmt<FMT_E4M3>(a, nullptr, s)
                           : launch_rowscaled_fmt<FMT_UE5M3>(a, nullptr, s);
}

hipError_t launch_quantize_pertoken(const QuantizeArgs& a, float* row_amax_out, hipStream_t s) {
  return a.fmt == FMT_E4M3 ? launch_rowscaled_fmt<FMT_E4M3>(a, row_amax_out, s)
                           : launch_rowscaled_fmt<FMT_UE5M3>(a, row_amax_out, s);
}

// ---------------------------------------------------------------- transformed blocks
// Quantization of the tensor with every block transformed by the 16-point
// random Hadamard transform first: row blocks through the one-lane-per-block
// stream, column blocks through the strip walker (column-wise only).
template <int FMT, int SELECT, int ROUND, bool WIDE>
static hipError_t launch_rht_typed(const QuantizeArgs& a, uint32_t signs, hipStream_t s) {
  const uint32_t key0 = sr_key(a.seed, 0u);
  const int cus = device_cu_count();
  if (a.axes == AXIS_ROW) {
    const int64_t nblocks = a.rows * a.cols / 16;
    const int64_t ngroups = (nblocks + 63) / 64;
    constexpr int B = kThreads;
    const int64_t grid = cap_grid((ngroups + B / 64 - 1) / (B / 64), (int64_t)cus * 8);
    hipLaunchKernelGGL((quantize_blocks_rht_kernel<FMT, SELECT, ROUND, WIDE, B>),
                       dim3((unsigned)grid), dim3(B), 0, s, reinterpret_cast<const uint4*>(a.x),
                       nblocks, a.amax, a.sg, a.seed, key0, reinterpret_cast<uint2*>(a.codes),
                       a.scales, a.count4, a.ws, signs);
    return hipGetLastError();
  }
  constexpr auto kern = quantize_tiles_kernel<FMT, SELECT, ROUND, WIDE, false, true, false, true>;
  int64_t grid, seg;
  walker_shape<kern>(a, grid, seg);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), 0, s, a.x, a.rows, a.cols, a.amax,
                     a.sg, a.seed, key0, a.codes, a.scales, a.codes_t, a.scales_t, a.count4, a.ws,
                     seg, signs);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_rht_fmt(const QuantizeArgs& a, uint32_t signs, hipStream_t s) {
  if (a.rounding == ROUND_SR) {
    const bool wide = (uint64_t)a.rows * (uint64_t)a.cols > (1ull << 32);
    return wide ? launch_rht_typed<FMT, SELECT_6, ROUND_SR, true>(a, signs, s)
                : launch_rht_typed<FMT, SELECT_6, ROUND_SR, false>(a, signs, s);
  }
  switch (a.select) {
    case SELECT_4OVER6: return launch_rht_typed<FMT, SELECT_4OVER6, ROUND_RNE, false>(a, signs, s);
    case SELECT_4OVER6_MAE: return launch_rht_typed<FMT, SELECT_4OVER6_MAE, ROUND_RNE, false>(a, signs, s);
    case SELECT_4OVER6_MAXERR: return launch_rht_typed<FMT, SELECT_4OVER6_MAXERR, ROUND_RNE, false>(a, signs, s);
    case SELECT_SWEEP: return launch_rht_typed<FMT, SELECT_SWEEP, ROUND_RNE, false>(a, signs, s);
    default: return launch_rht_typed<FMT, SELECT_6, ROUND_RNE, false>(a, signs, s);
  }
}

hipError_t launch_quantize_rht(const QuantizeArgs& a, uint32_t signs, hipStream_t s) {
  return a.fmt == FMT_E4M3 ? launch_rht_fmt<FMT_E4M3>(a, signs, s) : launch_rht_fmt<FMT_UE5M3>(a, signs, s);
}

template <int FMT>
static hipError_t launch_2d_fmt(const QuantizeArgs& a, hipStream_t s) {
  constexpr auto kBoth = quantize_tiles_kernel<FMT, SELECT_6, ROUND_RNE, false, true, true, true>;
  constexpr auto kRow = quantize_tiles_kernel<FMT, SELECT_6, ROUND_RNE, false, true, false, true>;
  const bool both = a.axes == (AXIS_ROW | AXIS_COL);
  int64_t grid, seg;
  if (both) walker_shape<kBoth>(a, grid, seg);
  else walker_shape<kRow>(a, grid, seg);
  hipLaunchKernelGGL(both ? kBoth : kRow, dim3((unsigned)grid), dim3(kThreads), 0, s, a.x, a.rows,
                     a.cols, a.amax, a.sg, a.seed, 0u, a.codes, a.scales, a.codes_t, a.scales_t,
                     nullptr, nullptr, seg, 0u);
  return hipGetLastError();
}

hipError_t launch_quantize_2d(const QuantizeArgs& a, hipStream_t s) {
  return a.fmt == FMT_E4M3 ? launch_2d_fmt<FMT_E4M3>(a, s) : launch_2d_fmt<FMT_UE5M3>(a, s);
}

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t s) {
  if (a.fmt == FMT_E4M3) return launch_fmt<FMT_E4M3>(a, s);
  return launch_fmt<FMT_UE5M3>(a, s);
}

}  // namespace nvfp4
