// OCP MXFP4 element and block arithmetic shared by the MXFP4 kernels and the AWQ
// search. Page quantize_dflash_mxfp4.py: the E2M1 table and quantize_mxfp4.
#pragma once

#include "device_common.hpp"

namespace gwb {

// e8m0 byte of a 32-block from its amax (float32, >= 0): exponent e = floor(log2 amax)
// - 2 (exact, from the bits), 0 for an all-zero block, clamped to >= -127 (amax is
// finite, so e <= 125); e8m0 = e + 127.
__device__ __forceinline__ uint32_t mx_e8m0(float amax) {
  uint32_t E = __float_as_uint(amax) >> 23;       // biased exponent; 0 for subnormals
  uint32_t e8 = E >= 2u ? E - 2u : 0u;            // E - 127 - 2 + 127, clamped at -127
  return amax == 0.0f ? 127u : e8;
}
// 2**-e as a float32 (always a normal number for e8m0 in [0, 252]).
__device__ __forceinline__ float mx_inv_scale(uint32_t e8m0) {
  return __uint_as_float((254u - e8m0) << 23);
}

// e2m1 code of x for a block with inverse scale 2**-e: v = x * 2**-e (exact unless v
// is subnormal, which is far below the first rounding threshold), m = min(|v|, 6),
// rounded half-to-even onto the e2m1 grid by adding and removing a power of two whose
// float32 ulp equals the grid spacing at m (0.5 below 2, 1 on [2, 4), 2 on [4, 6]);
// the index is then read from the exponent and top mantissa bit of the result.
// The sign bit is x's (so -0.0 and negatives that round to 0 give code 8).
__device__ __forceinline__ float e2m1_round_mag(float v) {
  float m = fminf(fabsf(v), 6.0f);
  uint32_t mexp = __float_as_uint(m) & 0x7F800000u;
  uint32_t big = (mexp > 0x3F800000u ? mexp : 0x3F800000u) + (22u << 23);
  float M = __uint_as_float(big);
  return (m + M) - M;                               // one of 0, .5, 1, 1.5, 2, 3, 4, 6
}
__device__ __forceinline__ uint32_t e2m1_index(float r) {
  uint32_t ub = __float_as_uint(r) >> 22;          // 0, 252(.5), 254(1) ... 259(6)
  return ub >= 254u ? ub - 252u : (ub == 252u ? 1u : 0u);
}
__device__ __forceinline__ uint32_t e2m1_code(float x, float inv_scale) {
  return e2m1_index(e2m1_round_mag(x * inv_scale)) | ((__float_as_uint(x) >> 31) << 3);
}

// Dequantized float32 of a 4-bit code with e8m0 scale: +-E2M1[c & 7] * 2**(e8m0-127).
// The magnitude's float32 bits are (idx + 252) << 22 for idx >= 2, 0.5 for idx 1.
__device__ __forceinline__ float e2m1_value(uint32_t c, float scale) {
  uint32_t idx = c & 7u;
  uint32_t mb = idx >= 2u ? (idx + 252u) << 22 : (idx == 1u ? 0x3F000000u : 0u);
  mb |= (c & 8u) << 28;
  return __uint_as_float(mb) * scale;
}
__device__ __forceinline__ float mx_scale(uint32_t e8m0) {
  return __uint_as_float(e8m0 ? e8m0 << 23 : 0x00400000u);   // 2**-127 is subnormal
}

}  // namespace gwb
