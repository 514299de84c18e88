// mm3_device.h -- device-side helpers shared by the gfx950 kernels.
//
// Vector types for MFMA operands, thin wrappers over the CDNA4 bf16 MFMA
// builtins, and the order-preserving float -> u32 map the selector uses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mm3 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 128;    // tokens per sparse block == tokens per page
constexpr int kDim = 128;      // index head dimension
constexpr int kWave = 64;      // CDNA wavefront

// D(16x16) += A(16x32) * B(32x16), bf16 in, fp32 accumulate.  Lane l holds
// A row l%16 / B column l%16 and 8 consecutive k of k-group l/16; D lane l
// holds column l%16, rows 4*(l/16) + 0..3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(32x32) += A(32x16) * B(16x32).  Lane l holds A row l%32 / B column l%32
// and 8 k of k-group l/32; D lane l holds column l%32 and, in register i,
// row 8*(i/4) + 4*(l/32) + i%4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Monotone map from finite fp32 to u32 (a < b  <=>  key(a) < key(b)), with
// -0 canonicalised to +0 so that the two compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Key of a forced (init / local) block: above every finite score.
constexpr uint32_t kForcedKey = 0xFFFFFFFFu;

// max(v, v of lane l ^ 16) and max(v, v of lane l ^ 32), without an LDS
// round trip.  The gfx950 lane-swap instructions exchange the odd 16-lane
// rows of one copy of v with the even rows of another (permlane16_swap), or
// the upper 32 lanes of one with the lower 32 of the other (permlane32_swap);
// afterwards each lane holds its own value in one copy and its partner's in
// the other, so the max of the two copies is the pairwise max.
__device__ __forceinline__ float wave_max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace mm3
