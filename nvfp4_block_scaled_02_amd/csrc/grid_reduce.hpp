// grid_reduce.hpp -- one value per workgroup combined across the grid in a
// fixed order, in the same launch, with no clearing kernel and no
// floating-point atomics.
//
// Every workgroup stores its value into its own 8-byte slot of a workspace
// and then arrives at one of kGroups counters (workgroup b at counter b mod
// kGroups, each counter on its own 128-byte line, so that same-address
// atomics queue kGroups ways in parallel instead of all on one address).  The
// last workgroup of a counter resets it and arrives at a top counter; the
// last workgroup at the top counter resets that one too and combines slots 0,
// 1, ..., G-1.  The combination is a fixed shape (a strided sequential pass
// per lane, a fixed DPP exchange pattern per wavefront, wavefronts in index order), so a
// floating-point sum depends only on G and the workgroup size, not on the
// order in which workgroups finished.
//
// Workspace contract: kWorkspaceBytes of device memory whose counters are
// zero before a launch; every launch that runs to completion leaves them
// zero.  Launches that use one workspace must not overlap.
//
// Ordering without cache maintenance: every access to a slot or a counter is
// a device-scope atomic read-modify-write, performed where the address is
// coherent for the whole GPU (all XCDs).  A workgroup publishes its slot with
// an exchange and arrives only after the exchange has returned (so it has
// been performed); the last workgroup reads the slots with read-modify-writes
// after its own arrival has returned.  No release or acquire fence is needed,
// so no XCD's L2 is written back or invalidated (a fence per workgroup costs
// microseconds when the kernel's outputs are still dirty in L2).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace nvfp4 {

constexpr int kSlots = 8192;                 // largest grid a reducing launch may use
constexpr int kGroups = 8;                   // arrival counters below the top counter
constexpr int kCtrStride = 32;               // uint32 words between counters (128 bytes)
constexpr size_t kCtrOffset = (size_t)kSlots * 8;
constexpr size_t kWorkspaceBytes = kCtrOffset + (size_t)(kGroups + 1) * kCtrStride * 4;

// Called by exactly one thread of every workgroup of the grid, once.  Returns
// true in the last workgroup to arrive; in it every slot [0, gridDim.x) holds
// its workgroup's value.
__device__ __forceinline__ bool grid_arrive(uint8_t* ws, uint64_t value) {
  const uint32_t G = gridDim.x, b = blockIdx.x;
  uint64_t* slots = reinterpret_cast<uint64_t*>(ws);
  uint32_t* ctr = reinterpret_cast<uint32_t*>(ws + kCtrOffset);
  const uint64_t prev = __hip_atomic_exchange(&slots[b], value, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
  // consume the exchange's result: the arrival below is issued only once the
  // exchange has returned
  __asm__ volatile("" :: "v"((uint32_t)prev), "v"((uint32_t)(prev >> 32)) : "memory");
  const uint32_t grp = b % kGroups;
  const uint32_t gsize = G / kGroups + (grp < G % kGroups ? 1u : 0u);
  const uint32_t ngroups = G < (uint32_t)kGroups ? G : (uint32_t)kGroups;
  uint32_t* gc = ctr + grp * kCtrStride;
  if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != gsize - 1)
    return false;
  // every member of this group has arrived: no further update in this launch
  __hip_atomic_exchange(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t* top = ctr + kGroups * kCtrStride;
  if (__hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != ngroups - 1)
    return false;
  __hip_atomic_exchange(top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Slot i, read with a read-modify-write (adds 0) where it is coherent.
__device__ __forceinline__ uint64_t slot_load(uint8_t* ws, uint32_t i) {
  return __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(ws) + i, (uint64_t)0, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
}

// The combinations: an identity, a binary operation, and the slot encoding.
struct SumU64 {
  typedef uint64_t T;
  static __device__ T identity() { return 0; }
  static __device__ T op(T a, T b) { return a + b; }
  static __device__ uint64_t to_bits(T v) { return v; }
  static __device__ T from_bits(uint64_t v) { return v; }
};
struct SumU32 {
  typedef uint32_t T;
  static __device__ T identity() { return 0; }
  static __device__ T op(T a, T b) { return a + b; }
  static __device__ uint64_t to_bits(T v) { return v; }
  static __device__ T from_bits(uint64_t v) { return (uint32_t)v; }
};
struct MaxU32 {
  typedef uint32_t T;
  static __device__ T identity() { return 0; }
  static __device__ T op(T a, T b) { return a > b ? a : b; }
  static __device__ uint64_t to_bits(T v) { return v; }
  static __device__ T from_bits(uint64_t v) { return (uint32_t)v; }
};
struct SumF64 {
  typedef double T;
  static __device__ T identity() { return 0.0; }
  static __device__ T op(T a, T b) { return a + b; }
  static __device__ uint64_t to_bits(T v) { return __builtin_bit_cast(uint64_t, v); }
  static __device__ T from_bits(uint64_t v) { return __builtin_bit_cast(double, v); }
};

// The wavefront's combination, in every lane: inside each row of 16 lanes an
// exchange at lane distance 1, 2, 4 and 8 (DPP moves; the operation is
// commutative, so both lanes of a pair hold the same bits), then the four
// row values in order.  No LDS round trip (a __shfl_xor butterfly costs one
// ds_bpermute per step: same-box A/B, the tensor amax 13.64 -> 13.43 us at
// 8192x4096 and 4.06 -> 3.78 us at 256x1024, the counting 4/6 quantizer at
// 4096x4096 10.58 -> 10.38 us, dequantize + error report 40.94 -> 40.47 us).
// Every lane of the wavefront must be active.
template <class R, int D>
__device__ __forceinline__ typename R::T xor_lane(typename R::T v) {
  typedef typename R::T T;
  if constexpr (sizeof(T) == 8) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = xor_lane_u32<D>((uint32_t)u), hi = xor_lane_u32<D>((uint32_t)(u >> 32));
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  } else {
    return __builtin_bit_cast(T, xor_lane_u32<D>(__builtin_bit_cast(uint32_t, v)));
  }
}

template <class R>
__device__ __forceinline__ typename R::T read_lane(typename R::T v, int lane) {
  typedef typename R::T T;
  if constexpr (sizeof(T) == 8) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  } else {
    return __builtin_bit_cast(T, (uint32_t)__builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
  }
}

template <class R>
__device__ __forceinline__ typename R::T wave_reduce(typename R::T v) {
  v = R::op(v, xor_lane<R, 1>(v));
  v = R::op(v, xor_lane<R, 2>(v));
  v = R::op(v, xor_lane<R, 4>(v));
  v = R::op(v, xor_lane<R, 8>(v));
  return R::op(R::op(R::op(read_lane<R>(v, 0), read_lane<R>(v, 16)), read_lane<R>(v, 32)),
               read_lane<R>(v, 48));
}

// Every thread of every workgroup calls this once with its own value (all
// threads must reach it: it holds workgroup barriers).  The workgroup's
// values are combined (wave_reduce, wavefronts in order), the grid's
// workgroup values are combined by the last workgroup, and true is returned
// to thread 0 of that workgroup with the grid total in *total.
template <class R, int BLOCK>
__device__ __forceinline__ bool grid_reduce(uint8_t* ws, typename R::T v, typename R::T* total) {
  typedef typename R::T T;
  static_assert(BLOCK % 64 == 0 && BLOCK <= 1024, "whole wavefronts");
  __shared__ T red[BLOCK / 64];
  __shared__ bool last;
  v = wave_reduce<R>(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    T t = red[0];
    for (int i = 1; i < BLOCK / 64; ++i) t = R::op(t, red[i]);
    last = grid_arrive(ws, R::to_bits(t));
  }
  __syncthreads();
  if (!last) return false;
  // the last workgroup: lane t takes slots t, t + BLOCK, ... in order
  T acc = R::identity();
  for (uint32_t i = threadIdx.x; i < gridDim.x; i += BLOCK) acc = R::op(acc, R::from_bits(slot_load(ws, i)));
  acc = wave_reduce<R>(acc);
  __syncthreads();  // red[] is reused
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x != 0) return false;
  T t = red[0];
  for (int i = 1; i < BLOCK / 64; ++i) t = R::op(t, red[i]);
  *total = t;
  return true;
}

// A grid sum of non-negative integers, at most 2^40 per launch (one per
// block of a tensor of at most 2^44 elements), added to *out.  Each
// workgroup's part travels inside its arrival: one 64-bit add of 2^41 + part
// to its group word (workgroup b at word b mod kGroups, each on its own
// 128-byte line; arrivals in the high 23 bits, which hold every grid of at
// most kSlots workgroups, the running sum in the low 41).  The last
// workgroup of a group resets the word and adds the group's sum to *out; the
// kGroups adds commute exactly (integers), so the total does not depend on
// the order in which groups finish.  A workgroup thus waits on one atomic
// round trip and the last of a group issues two atomics that return nothing.
// A second level (the groups' last workgroups arriving at a top word, whose
// last one adds the total) puts a second round trip at the end of the launch:
// same-box A/B, the counting 4/6 quantizer 10.21 -> 9.85 us at 4096x4096 and
// 16.62 -> 16.29 us at 8192x4096 without it; 32 groups instead of 8 were
// even with 8.  No slot is written or read.  The group words are the first
// kGroups counter lines of the workspace, viewed as 64-bit words (zero on
// entry, zero again on exit).  Every thread of every workgroup calls it once
// with its own part.
template <int BLOCK>
__device__ __forceinline__ void grid_count_add(uint8_t* ws, uint32_t part,
                                               unsigned long long* out) {
  static_assert(BLOCK % 64 == 0 && BLOCK <= 1024, "whole wavefronts");
  constexpr int kSumBits = 41;
  constexpr uint64_t kOne = 1ull << kSumBits, kLow = kOne - 1;
  static_assert(kSlots < (1 << (64 - kSumBits)), "arrivals fit above the sum");
  __shared__ uint32_t red[BLOCK / 64];
  part = wave_reduce<SumU32>(part);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = part;
  __syncthreads();
  if (threadIdx.x != 0) return;
  uint64_t t = 0;
  for (int i = 0; i < BLOCK / 64; ++i) t += red[i];
  const uint32_t G = gridDim.x, b = blockIdx.x;
  uint64_t* words = reinterpret_cast<uint64_t*>(ws + kCtrOffset);
  const uint32_t grp = b % kGroups;
  const uint32_t gsize = G / kGroups + (grp < G % kGroups ? 1u : 0u);
  uint64_t* gw = words + grp * (kCtrStride / 2);
  const uint64_t g = __hip_atomic_fetch_add(gw, kOne + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((g >> kSumBits) != gsize - 1) return;
  // every member of this group has arrived: no further update in this launch
  __hip_atomic_exchange(gw, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t gsum = (g & kLow) + t;
  if (gsum != 0) atomicAdd(out, (unsigned long long)gsum);
}

}  // namespace nvfp4
