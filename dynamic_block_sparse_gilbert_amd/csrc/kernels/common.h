// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dbs {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// float -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats -> packed bf16x2 (lo = a, hi = b).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Butterfly exchange across lanes (lane ^ mask) within a 64-wide wavefront.
__device__ __forceinline__ float xor_shfl(float v, int mask) {
  const int lane = threadIdx.x & 63;
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(v)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr int kXcdRanges = 8;   // XCDs of an MI355X; workgroups are dealt to them round-robin

// Range x of the split of `total` logical ids into kXcdRanges contiguous
// ranges (the first total % 8 ranges one longer).
__device__ __forceinline__ void xcd_range(int x, int total, int& start, int& size) {
  const int per = total / kXcdRanges, rem = total % kXcdRanges;
  start = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  size = per + (x < rem ? 1 : 0);
}

// Remap a linear workgroup id so that the hardware's round-robin placement
// over the XCDs gives every XCD one contiguous range of logical ids (work
// items that share K/V then share that XCD's L2).
__device__ __forceinline__ int xcd_remap(int wg, int total) {
  const int per = total / kXcdRanges, rem = total % kXcdRanges;
  const int xcd = wg % kXcdRanges, slot = wg / kXcdRanges;
  return (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

}  // namespace dbs
