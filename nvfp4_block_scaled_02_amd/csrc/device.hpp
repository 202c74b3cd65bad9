// device.hpp -- gfx950 device helpers shared by the NVFP4 kernels: bf16
// unpacking, block-scale encoders, E2M1 conversion, the stochastic-rounding
// counter hash, and cross-lane moves.  Device code only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- streaming
// Non-temporal (streaming) global loads and stores: every byte is touched
// once, so they should not displace anything from the caches.
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 ld_nt(const uint2* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ float4 ld_nt(const float4* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t ld_nt(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(float4 v, float4* p) {
  f32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void st_nt(uint4 v, uint4* p) {
  u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void st_nt(uint2 v, uint2* p) {
  u32x2 w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void st_nt(uint32_t v, uint32_t* p) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void st_nt(uint8_t v, uint8_t* p) { __builtin_nontemporal_store(v, p); }

// ---------------------------------------------------------------- bf16
// A dword holds two bf16 patterns, the lower-addressed element in the low
// half.  Widening is exact: the pattern moves to the high half of a float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Largest |bf16| bit pattern (sign cleared) of the 8 values in a 16-byte
// chunk, as an integer: for non-NaN patterns integer order is magnitude
// order, and every NaN pattern exceeds +inf (0x7F80).
__device__ __forceinline__ uint32_t chunk_abs_max_bits(uint4 w) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const uint32_t m = 0x7FFF7FFFu;
  uint32_t a = w.x & m, b = w.y & m, c = w.z & m, d = w.w & m;
  u16x2 va = __builtin_bit_cast(u16x2, a), vb = __builtin_bit_cast(u16x2, b);
  u16x2 vc = __builtin_bit_cast(u16x2, c), vd = __builtin_bit_cast(u16x2, d);
  u16x2 ab = __builtin_elementwise_max(va, vb);
  u16x2 cd = __builtin_elementwise_max(vc, vd);
  u16x2 r = __builtin_elementwise_max(ab, cd);
  uint32_t lo = r[0], hi = r[1];
  return lo > hi ? lo : hi;
}

// ---------------------------------------------------------------- cross-lane
// Value of the lane whose index differs in bit 0 (quad_perm [1,0,3,2]).
__device__ __forceinline__ uint32_t xor1_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ float xor1_f32(float v) {
  return __uint_as_float(xor1_u32(__float_as_uint(v)));
}

// Value of the lane whose index differs in bit 1, 2 or 3 (inside each row of
// 16 lanes): quad_perm [2,3,0,1]; row_half_mirror (lane l <- l ^ 7 inside its
// 8) then quad_perm [3,2,1,0] (l ^ 3); row_ror:8 (a rotation by half a row).
__device__ __forceinline__ uint32_t xor2_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t xor4_u32(uint32_t v) {
  const int m = __builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);
  return (uint32_t)__builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t xor8_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);
}
template <int D>
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t v) {
  if constexpr (D == 1) return xor1_u32(v);
  else if constexpr (D == 2) return xor2_u32(v);
  else if constexpr (D == 4) return xor4_u32(v);
  else return xor8_u32(v);
}

// Within each group of 4 lanes, lane k receives lane k-1's value (lane 0
// keeps its own): quad_perm [0,0,1,2].
__device__ __forceinline__ double shift1_in_quad_f64(double v) {
  uint64_t u = __builtin_bit_cast(uint64_t, v);
  uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, 0x90, 0xF, 0xF, false);
  uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), 0x90, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------- E2M1
// gfx950 v_cvt_scalef32_pk_fp4_f32 with a unit scale is round-to-nearest-
// even onto E2M1 with saturation at +-6 and the sign of zero kept, for every
// non-NaN binary32 input (checked exhaustively against the CPU reference).
// Byte `sel` of `old` receives {b:a} (a in the low nibble).
#define NVFP4_CVT_PK_FP4(old, a, b, sel) __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((old), (a), (b), 1.0f, (sel))
// Exact decode of byte `sel` of a packed word into {low nibble, high nibble}.
#define NVFP4_DEC_PK_FP4(word, sel) __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((word), 1.0f, (sel))

// Workgroup barrier that orders LDS only: fences scoped to the workgroup and
// to the local (LDS) address space wait for this wavefront's LDS operations
// (lgkmcnt) but not for its global loads, so loads issued before the barrier
// stay in flight across it (__syncthreads() would wait for them).  Global
// memory is not ordered by it.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A register with no defined value, for destinations whose every byte is
// written before use (the empty asm emits nothing, so no copy is made).
__device__ __forceinline__ uint32_t scratch_vgpr() {
  uint32_t w;
  asm volatile("" : "=v"(w));
  return w;
}

// 8 binary32 values -> one dword of 8 nibbles, element i in nibble i.
__device__ __forceinline__ uint32_t e2m1_rne_pack8(const float (&y)[8]) {
  uint32_t w = scratch_vgpr();  // placeholder: all four bytes are written
  w = NVFP4_CVT_PK_FP4(w, y[0], y[1], 0);
  w = NVFP4_CVT_PK_FP4(w, y[2], y[3], 1);
  w = NVFP4_CVT_PK_FP4(w, y[4], y[5], 2);
  w = NVFP4_CVT_PK_FP4(w, y[6], y[7], 3);
  return w;
}

__device__ __forceinline__ void e2m1_unpack8(uint32_t w, float (&q)[8]) {
  f32x2 a = NVFP4_DEC_PK_FP4(w, 0), b = NVFP4_DEC_PK_FP4(w, 1);
  f32x2 c = NVFP4_DEC_PK_FP4(w, 2), d = NVFP4_DEC_PK_FP4(w, 3);
  q[0] = a[0]; q[1] = a[1]; q[2] = b[0]; q[3] = b[1];
  q[4] = c[0]; q[5] = c[1]; q[6] = d[0]; q[7] = d[1];
}

// ---------------------------------------------------------------- SR
// MurmurHash3 fmix32 finalizer (A. Appleby, public domain).
__host__ __device__ inline uint32_t fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}

// fmix32 after its first step: fmix32(h) == fmix32_tail(h ^ (h >> 16)).
// For the 8 inputs b ^ i (i < 8) of one chunk the first step is shared:
// (b ^ i) ^ ((b ^ i) >> 16) == (b ^ (b >> 16)) ^ i.
__device__ __forceinline__ uint32_t fmix32_tail(uint32_t h) {
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  // h ^ (h >> 16) in one instruction: SDWA reads the high half-word of the
  // first operand, zero-extended (the compiler otherwise emits shift + xor)
  uint32_t r;
  asm("v_xor_b32_sdwa %0, %1, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1 src1_sel:DWORD"
      : "=v"(r) : "v"(h));
  return r;
}

// Key of the counter hash for indices sharing the high word idx_hi.
__host__ __device__ inline uint32_t sr_key(uint64_t seed, uint32_t idx_hi) {
  uint32_t h = (uint32_t)(seed >> 32) ^ idx_hi ^ 0x9E3779B9u;
  // fmix32 spelled out so the host can form the key too
  h ^= h >> 16; h *= 0x85ebca6bu; h ^= h >> 13; h *= 0xc2b2ae35u; h ^= h >> 16;
  h ^= (uint32_t)seed;
  h ^= h >> 16; h *= 0x85ebca6bu; h ^= h >> 13; h *= 0xc2b2ae35u; h ^= h >> 16;
  return h;
}

// Stochastic rounding onto E2M1 with gfx950 v_cvt_scalef32_sr_pk_fp4_f32
// (unit scale) on a pair (a, b) of binary32 values in consecutive registers.
// Measured rule: a (low nibble) goes up iff (r >> 10) + floor(p * 2^22) >=
// 2^22, p = (|a| - lo) / (hi - lo), r the random word; b (high nibble) uses
// bits [9, 31) of r instead; |v| >= 6 saturates; the sign is kept.  So that
// every element sees only its own hash h (variate h >> 10), each pair is
// converted twice: with r = h_even (its low nibble kept) and with r = h_odd >> 1
// (its high nibble kept); one bitfield select merges the two words.
//
// The instruction writes only the selected byte of its destination and keeps
// the other three (checked on the hardware), but the compiler's builtin for
// it does not tie the destination to the `old` operand; it is therefore
// issued here as inline assembly with a read-write destination.
template <int SEL>
__device__ __forceinline__ uint32_t sr_fp4_into(uint32_t old, f32x2 v, uint32_t r) {
  if constexpr (SEL == 0)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0" : "+v"(old) : "v"(v), "v"(r));
  else if constexpr (SEL == 1)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,0]" : "+v"(old) : "v"(v), "v"(r));
  else if constexpr (SEL == 2)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,0,1]" : "+v"(old) : "v"(v), "v"(r));
  else
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,1]" : "+v"(old) : "v"(v), "v"(r));
  return old;
}

// Packs 8 elements (pairs yp[b] = elements 2b, 2b+1) with their hashes.
// we / wo: placeholder words (every byte is overwritten; pass registers that
// are dead, e.g. the bits of consumed inputs, to avoid copies).
__device__ __forceinline__ uint32_t e2m1_sr_pack8(const f32x2 (&yp)[4], const uint32_t (&h)[8],
                                                  uint32_t we, uint32_t wo) {
  we = sr_fp4_into<0>(we, yp[0], h[0]);
  wo = sr_fp4_into<0>(wo, yp[0], h[1] >> 1);
  we = sr_fp4_into<1>(we, yp[1], h[2]);
  wo = sr_fp4_into<1>(wo, yp[1], h[3] >> 1);
  we = sr_fp4_into<2>(we, yp[2], h[4]);
  wo = sr_fp4_into<2>(wo, yp[2], h[5] >> 1);
  we = sr_fp4_into<3>(we, yp[3], h[6]);
  wo = sr_fp4_into<3>(wo, yp[3], h[7] >> 1);
  return (we & 0x0F0F0F0Fu) | (wo & 0xF0F0F0F0u);
}

// ---------------------------------------------------------------- scales
// Block-scale encoders: nearest finite code value, ties to the even code,
// saturating at the largest finite code; s >= 0 (+inf saturates).  NaN is
// handled by the caller.
//
// E4M3 (both candidates at once): gfx950 v_cvt_scalef32_pk_fp8_f32 is OCP
// E4M3 round-to-nearest-even for every input up to 464 and gives NaN above,
// so the inputs are first clamped to 448 (which is also the nearest code for
// everything above 448).  Low byte = a, next byte = b.  The sign bits are
// dropped: for the non-negative inputs of the method they are 0, and a
// negative input (only from an unusable amax, whose output is replaced by the
// NaN code) must still index inside the 127-entry code table.
__device__ __forceinline__ uint32_t e4m3_encode_pair(float a, float b) {
  i16x2 old = __builtin_bit_cast(i16x2, __float_as_uint(a));  // low word is replaced
  i16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(old, __builtin_fminf(a, 448.0f),
                                                     __builtin_fminf(b, 448.0f), 1.0f, false);
  return (uint32_t)(uint16_t)r[0] & 0x7F7Fu;
}

// UE5M3 (bias 15, subnormal step 2^-17, largest finite 0xFE = 114688):
// integer round-to-nearest-even of the binary32 significand to 3 bits.
__device__ __forceinline__ uint32_t ue5m3_encode(float s) {
  const uint32_t b = __float_as_uint(s);
  const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
  const uint32_t normal = (r >> 20) - (112u << 3);
  const uint32_t sub = (uint32_t)__builtin_rintf(s * 0x1p17f);
  uint32_t code = s < 0x1p-14f ? sub : normal;
  return code > 0xFEu ? 0xFEu : code;
}

__device__ __forceinline__ uint32_t encode_pair(int fmt, float a, float b) {
  if (fmt == FMT_E4M3) return e4m3_encode_pair(a, b);
  return ue5m3_encode(a) | (ue5m3_encode(b) << 8);
}

// Exact value of a non-negative finite scale code as binary32.
__device__ __forceinline__ float decode_scale(int fmt, uint32_t code) {
  const uint32_t m = code & 7u;
  if (fmt == FMT_E4M3) {
    const uint32_t e = (code & 0x7Fu) >> 3;  // bit 7 is the sign
    float sub = (float)m * 0x1p-9f;
    float nrm = __uint_as_float(((code & 0x7Fu) << 20) + (120u << 23));
    float v = e == 0 ? sub : nrm;
    v = (code & 0x7Fu) == 0x7Fu ? __builtin_nanf("") : v;
    return (code & 0x80u) ? -v : v;
  }
  const uint32_t e = code >> 3;
  float sub = (float)m * 0x1p-17f;
  float nrm = __uint_as_float((code << 20) + (112u << 23));
  float v = e == 0 ? sub : nrm;
  return code == 0xFFu ? __builtin_nanf("") : v;
}

// Per-tensor constants derived from the device amax, binary32:
//   alpha = A / (6 S_g)  (1 if A = 0; NaN if A < 0 or non-finite)
//   K_Q   = 1 / (Q alpha), +inf replaced by FLT_MAX.
struct TensorScale {
  float alpha, k6, k4;
  bool nan;
};

// Outer scale alpha = A / (6 S_g) (1 for A = 0); NaN when A is negative or
// not finite (no usable scale).
__device__ __forceinline__ float outer_alpha(float amax, float sg) {
  if (!(amax >= 0.0f) || __builtin_isinf(amax)) return __builtin_nanf("");
  return amax == 0.0f ? 1.0f : amax / (6.0f * sg);
}

__device__ __forceinline__ TensorScale tensor_scale(float amax, float sg) {
  TensorScale t;
  t.nan = !(amax >= 0.0f) || __builtin_isinf(amax);
  t.alpha = amax == 0.0f ? 1.0f : amax / (6.0f * sg);
  float r6 = 1.0f / (6.0f * t.alpha);
  float r4 = 1.0f / (4.0f * t.alpha);
  t.k6 = __builtin_isinf(r6) ? 3.40282347e38f : r6;
  t.k4 = __builtin_isinf(r4) ? 3.40282347e38f : r4;
  return t;
}

// Table entry of code c: {S_EFF = D[c] * alpha, INV_S = 1 / S_EFF, or 0 if
// S_EFF = 0 or the reciprocal overflows}.
__device__ __forceinline__ f32x2 scale_entry(int fmt, uint32_t c, float alpha) {
  float s = decode_scale(fmt, c) * alpha;
  float r = s == 0.0f ? 0.0f : 1.0f / s;
  r = __builtin_isinf(r) ? 0.0f : r;
  f32x2 e;
  e[0] = s;
  e[1] = r;
  return e;
}

// ---------------------------------------------------------------- issue priority
// A SIMD issues from its oldest ready wavefront first, so of the workgroups
// that share a CU the one dispatched first runs ahead; once it has finished,
// the later one runs its remaining work at half the occupancy.  The
// persistent kernels counter that with the wavefront issue priority: the
// later-dispatched half of the grid starts one level above the earlier half,
// and every wavefront drops one level at each third of its workgroup's task
// list, so the workgroup that is ahead yields to the one that is behind.
// Same-box A/B on the one-lane-per-block quantizer (two 1024-lane workgroups
// per CU, steady-state timing, outputs identical): scale sweep 517 -> 507 us,
// SR row stream at 16384x8192 60.0 -> 59.5 us, counting 4/6 at 4096x4096
// 10.87 -> 10.68 us; the 4/6 quantizer at 8192x4096 even (15.9 us).  Only
// launches of two 1024-lane workgroups per CU use it: with more, smaller
// workgroups per CU the later half of the grid is not the later workgroup of
// each CU (the 256-lane transform quantizer ran 10% slower with it).  The
// dequantize + error-report stream, with the same launch shape and its trip
// count as the progress, ran 4% slower with it (40.8 -> 42.5 us) and does
// not use it.
struct ProgressPriority {
  uint64_t c1, c2, c3;  // tasks at which the level drops: ceil(kT/3), k = 1, 2, 3
  int top;              // level at task 0
  // tasks: about the number of tasks of one workgroup (T above)
  __device__ explicit ProgressPriority(uint64_t tasks) {
    const uint64_t T = tasks > 0 ? tasks : 1;
    c1 = (T + 2) / 3;
    c2 = (2 * T + 2) / 3;
    c3 = T;
    top = 2 + (blockIdx.x >= gridDim.x / 2 ? 1 : 0);
  }
  // sets the calling wavefront's priority for its task `task` (uniform)
  __device__ __forceinline__ void set(uint64_t task) const {
    const int v = top - (task >= c1 ? 1 : 0) - (task >= c2 ? 1 : 0) - (task >= c3 ? 1 : 0);
    if (v >= 3) asm volatile("s_setprio 3");
    else if (v == 2) asm volatile("s_setprio 2");
    else if (v == 1) asm volatile("s_setprio 1");
    else asm volatile("s_setprio 0");
  }
};

}  // namespace nvfp4
