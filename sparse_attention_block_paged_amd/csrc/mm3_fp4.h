// mm3_fp4.h -- NVFP4 index-K element decode shared by the scorers.
//
// Key element value = e4m3_rn_satfinite(e2m1(nibble) * e4m3(scale)) (page
// "vllm.models.minimax_m3.amd.indexer_nvfp4", module docstring).  For every
// scale byte the table holds the E4M3 codes of the 8 non-negative E2M1
// magnitudes times that scale, rounded to nearest-even and saturated at 448;
// the nibble's sign is XORed in at run time.  Built at compile time (each
// translation unit keeps its own copy of the 2 KiB table).
#pragma once

#include "mm3_device.h"

namespace mm3 {

struct Fp4Lut {
  uint32_t w[256][2];
};

// e4m3 value of a non-negative code, in units of 2^-9
constexpr int64_t e4m3_units9(int c) {
  int e = (c >> 3) & 15, m = c & 7;
  return e == 0 ? m : (int64_t)(8 + m) << (e - 1);
}

// E4M3 code (no sign) nearest to p * 2^-10, ties to even code, saturating.
constexpr int e4m3_code_from_units10(int64_t p) {
  int code = 0;
  if (p < 16) {  // below the smallest normal: grid step 2 units
    int64_t q = p >> 1;
    if (p & 1) q += (q & 1);
    code = (int)q;
  } else {
    int lg = 0;
    while ((p >> (lg + 1)) != 0) ++lg;  // floor(log2 p) >= 4
    int e = lg - 3;                     // p in [2^(e+3), 2^(e+4)), step 2^e
    int64_t q = p >> e, rem = p & ((int64_t(1) << e) - 1), half = int64_t(1) << (e - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
    code = (e << 3) + (int)(q - 8);
  }
  return code > 0x7E ? 0x7E : code;
}

constexpr Fp4Lut make_fp4_lut() {
  Fp4Lut t{};
  const int mag2[8] = {0, 1, 2, 3, 4, 6, 8, 12};  // e2m1 magnitudes x 2
  for (int s = 0; s < 256; ++s) {
    int a = s & 0x7F;
    uint32_t lo = 0, hi = 0;
    for (int j = 0; j < 8; ++j) {
      int code = 0;
      if (a != 0x7F)  // NaN scale: unspecified, mapped to +-0
        code = e4m3_code_from_units10(mag2[j] * e4m3_units9(a));
      code |= (s & 0x80);
      if (j < 4)
        lo |= (uint32_t)code << (8 * j);
      else
        hi |= (uint32_t)code << (8 * (j - 4));
    }
    t.w[s][0] = lo;
    t.w[s][1] = hi;
  }
  return t;
}

__device__ const Fp4Lut kFp4Lut = make_fp4_lut();

// 8 NVFP4 elements (one dword of nibbles, element 2i in the low nibble of
// byte i) -> 4 dwords of bf16 pairs in the element order
// {0,2 | 4,6 | 1,3 | 5,7}; tab = the 8 E4M3 codes for this group's scale.
__device__ __forceinline__ u32x4 fp4x8_to_bf16(uint32_t x, u32x2 tab) {
  uint32_t c_even = __builtin_amdgcn_perm(tab.y, tab.x, x & 0x07070707u) ^
                    ((x << 4) & 0x80808080u);
  uint32_t c_odd = __builtin_amdgcn_perm(tab.y, tab.x, (x >> 4) & 0x07070707u) ^
                   (x & 0x80808080u);
  u32x4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c_even, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c_even, 1.0f, true));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c_odd, 1.0f, false));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c_odd, 1.0f, true));
  return r;
}

// This thread's table entry (threads 0..255 one entry each).
__device__ __forceinline__ u32x2 lut_entry() {
  return u32x2{kFp4Lut.w[threadIdx.x][0], kFp4Lut.w[threadIdx.x][1]};
}

// Copy the table into LDS (threads 0..255 one entry each).
__device__ __forceinline__ void fill_lut(u32x2* lut) { lut[threadIdx.x] = lut_entry(); }

}  // namespace mm3
