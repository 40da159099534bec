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

// Streaming (non-temporal) 16-byte global accesses for data touched once:
// on gfx950 they lift copy bandwidth by ~5% over default-policy accesses.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(void* p, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ uint32_t ld_stream32(const uint32_t* p) {
  return __builtin_nontemporal_load(p);
}

}  // namespace wkv
