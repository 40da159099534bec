// Device helpers shared by the libwkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// float -> bf16 bits, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 b = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, b);
}

// Two floats -> packed bf16 pair (lo in bits 0..15), RNE.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  f32x2_t f = {lo, hi};
  bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

// Order-preserving map of a double onto uint64 (ascending doubles ->
// ascending keys). -0.0 is folded onto +0.0 and every NaN onto the largest
// key, so NaN orders after every number and equal values compare equal.
__device__ __forceinline__ uint64_t order_key(double s) {
  s = s + 0.0;
  if (s != s) return ~0ull;
  uint64_t u = __double_as_longlong(s);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

}  // namespace wkv
