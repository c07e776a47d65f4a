// OCP MXFP4 block arithmetic on gfx950, shared by the MXFP4 kernels and the AWQ search.
// Page quantize_dflash_mxfp4.py: the E2M1 table, quantize_mxfp4, dequantize_mxfp4.
//
// Element rounding uses CDNA4's scaled FP4 conversions (v_cvt_scalef32_pk_fp4_*,
// v_cvt_scalef32_pk_*_fp4). They divide (or multiply back) by a power-of-two scale and
// round to e2m1 half-to-even with saturation to 6 and the sign kept on zeros, which is
// exactly quantize_mxfp4's v = x / 2**e, sign = signbit(v), mag = min(|v|, 6), nearest
// magnitude with ties to the even code. This was checked on the device against an
// independent software rounding for every finite bf16 input under every E8M0 scale,
// random and near-tie float32 inputs, and every code byte on the way back.
#pragma once

#include "device_common.hpp"

namespace gwb {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// e8m0 byte of a 32-block from the float32 bits of its amax (>= 0):
// exponent e = floor(log2 amax) - 2 from the biased exponent field (exact, also for
// subnormals, which clamp), 0 for an all-zero block, clamped to >= -127 (a finite
// amax gives e <= 125); e8m0 = e + 127.
__device__ __forceinline__ uint32_t mx_e8m0_bits(uint32_t amax_bits) {
  uint32_t E = amax_bits >> 23;
  uint32_t e8 = E >= 2u ? E - 2u : 0u;
  return amax_bits == 0u ? 127u : e8;
}

// Scale operand of the conversions: the instruction reads the E8M0 byte from the
// float's exponent field, so 2**(e8m0 - 127) is passed as e8m0 << 23 (0.0 for 2**-127).
__device__ __forceinline__ float mx_scale_operand(uint32_t e8) { return __uint_as_float(e8 << 23); }

// |x| maximum of 8 bf16 (4 dwords) as float32 bits: bf16 magnitudes order like
// unsigned integers, so a packed 16-bit integer max does it.
__device__ __forceinline__ uint32_t absmax8_bits(U4 v) {
  const uint32_t m = 0x7FFF7FFFu;
  u16x2_t a = __builtin_bit_cast(u16x2_t, v.x & m), b = __builtin_bit_cast(u16x2_t, v.y & m);
  u16x2_t c = __builtin_bit_cast(u16x2_t, v.z & m), d = __builtin_bit_cast(u16x2_t, v.w & m);
  u16x2_t r = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  uint32_t lo = r[0], hi = r[1];
  return (lo > hi ? lo : hi) << 16;
}
__device__ __forceinline__ uint32_t absmax8_bits(const float* x) {
  float a = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
  float b = fmaxf(fmaxf(fabsf(x[4]), fabsf(x[5])), fmaxf(fabsf(x[6]), fabsf(x[7])));
  return __float_as_uint(fmaxf(a, b));
}
// Maximum over the 4 lanes of a 32-block (non-negative float bits order as integers).
__device__ __forceinline__ uint32_t quad_max_u(uint32_t x) {
  x = max(x, dpp_read_u<kDppXor1>(x));
  return max(x, dpp_read_u<kDppXor2>(x));
}

// 8 weights -> 8 codes in one word (code i in bits 4i..4i+3: byte j = code(2j) |
// code(2j+1) << 4, the packed layout).
__device__ __forceinline__ uint32_t mx_pack8(U4 v, float sc) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(bf16x2_t, v.x), sc, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2_t, v.y), sc, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2_t, v.z), sc, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2_t, v.w), sc, 3);
}
__device__ __forceinline__ uint32_t mx_pack8(const float* x, float sc) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[0], x[1], sc, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2], x[3], sc, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[4], x[5], sc, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[6], x[7], sc, 3);
}

// Dequantized value of one code with an E8M0 byte of 255, which the conversions do not
// define: the page's float32 product +-E2M1[c & 7] * 2**128 (inf, or NaN for 0 * inf).
__device__ __forceinline__ float mx_value_nan_scale(uint32_t c) {
  float mag = __uint_as_float((c & 7u) ? 0x7F800000u : 0x7FC00000u);
  return (c & 8u) ? -mag : mag;
}

// word of 8 codes -> 8 float32 / 8 bf16 (exact: e2m1 values times a power of two).
// mx_unpack8_cvt takes the scale operand of an E8M0 byte other than 255.
__device__ __forceinline__ void mx_unpack8_cvt(uint32_t w, float sc, float* d) {
  f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 0);
  f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 1);
  f32x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 2);
  f32x2_t e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 3);
  d[0] = a[0]; d[1] = a[1]; d[2] = b[0]; d[3] = b[1];
  d[4] = c[0]; d[5] = c[1]; d[6] = e[0]; d[7] = e[1];
}
__device__ __forceinline__ void mx_unpack8(uint32_t w, uint32_t e8, float* d) {
  if (e8 == 255u) {
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = mx_value_nan_scale((w >> (4 * i)) & 0xFu);
    return;
  }
  mx_unpack8_cvt(w, mx_scale_operand(e8), d);
}
__device__ __forceinline__ U4 mx_unpack8_bf16(uint32_t w, uint32_t e8) {
  if (e8 == 255u) {
    float d[8];
    mx_unpack8(w, e8, d);
    return U4{f32_to_bf16_rne(d[0]) | (f32_to_bf16_rne(d[1]) << 16), f32_to_bf16_rne(d[2]) | (f32_to_bf16_rne(d[3]) << 16),
              f32_to_bf16_rne(d[4]) | (f32_to_bf16_rne(d[5]) << 16), f32_to_bf16_rne(d[6]) | (f32_to_bf16_rne(d[7]) << 16)};
  }
  const float sc = mx_scale_operand(e8);
  return U4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3))};
}

}  // namespace gwb
