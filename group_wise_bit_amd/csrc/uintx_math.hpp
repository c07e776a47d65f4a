// Per-weight-dtype arithmetic of the affine uintx format. Page uintx_quant.py,
// UIntXQuantizer._quantize_impl / _dequantize_native: the ops run in the weight's own
// dtype, each one float32 op whose result is rounded to that dtype (bfloat16, float16;
// float32 weights: plain float32 ops), and the scale is stored as that dtype.
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace gwb {

// Storage word, rounding of a float32 result to the dtype, value of a stored word, the
// word of a value that is already of the dtype, and the 32-bit LDS word that carries
// (a scale or reciprocal of the dtype, a zero point) between the lanes of a group.
template <int DT> struct UxDt;
template <> struct UxDt<kBF16> {
  using T = uint16_t;
  using Lds = uint32_t;
  static __device__ __forceinline__ float rnd(float x) { return round_bf16(x); }
  static __device__ __forceinline__ float value(uint32_t h) { return __uint_as_float(h << 16); }
  static __device__ __forceinline__ T word(float v) { return (T)(__float_as_uint(v) >> 16); }
  static __device__ __forceinline__ Lds pack(uint32_t w, uint32_t zp) { return (w << 16) | zp; }
  static __device__ __forceinline__ float lds_value(Lds l) { return __uint_as_float(l & 0xFFFF0000u); }
  static __device__ __forceinline__ float lds_zp(Lds l) { return (float)(l & 0xFFu); }
};
template <> struct UxDt<kF16> {
  using T = uint16_t;
  using Lds = uint32_t;
  static __device__ __forceinline__ float rnd(float x) { return (float)(_Float16)x; }   // RNE, overflow to inf
  static __device__ __forceinline__ float value(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }
  static __device__ __forceinline__ T word(float v) { return __builtin_bit_cast(T, (_Float16)v); }
  static __device__ __forceinline__ Lds pack(uint32_t w, uint32_t zp) { return (w << 16) | zp; }
  static __device__ __forceinline__ float lds_value(Lds l) { return value(l >> 16); }
  static __device__ __forceinline__ float lds_zp(Lds l) { return (float)(l & 0xFFu); }
};
template <> struct UxDt<kF32> {
  using T = float;
  using Lds = uint2;
  static __device__ __forceinline__ float rnd(float x) { return x; }
  static __device__ __forceinline__ float value(float h) { return h; }
  static __device__ __forceinline__ T word(float v) { return v; }
  static __device__ __forceinline__ Lds pack(float w, uint32_t zp) { return make_uint2(__float_as_uint(w), zp); }
  static __device__ __forceinline__ float lds_value(Lds l) { return __uint_as_float(l.x); }
  static __device__ __forceinline__ float lds_zp(Lds l) { return (float)l.y; }
};

// Raw words of 8 consecutive weights: one 16-byte load for the 2-byte dtypes, two for
// float32 (Raw8 of device_common.hpp), widened to float32.
template <int DT>
__device__ __forceinline__ void ux_widen8(const Raw8<typename UxDt<DT>::T>& r, float* x) {
  if constexpr (DT == kF16) {
    const uint32_t w[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[2 * q] = UxDt<kF16>::value(w[q] & 0xFFFFu);
      x[2 * q + 1] = UxDt<kF16>::value(w[q] >> 16);
    }
  } else {
    to_f32(r, x);
  }
}

// Group qparams from the group's min and max: mn = min(min, 0), mx = max(max, 0);
// scale = r(r(mx - mn) / qmax), at least 2^-23; zp = clamp(-rint(r(mn / scale)), 0,
// qmax); inv = r(1 / scale), r the rounding to the weight dtype. The divisions are IEEE.
struct UxQP { float s, inv, zp; };
template <int DT>
__device__ __forceinline__ UxQP ux_qparams(float mn, float mx, float qmax) {
  using D = UxDt<DT>;
  const float mnn = fminf(mn, 0.0f), mxp = fmaxf(mx, 0.0f);
  const float s = fmaxf(D::rnd(D::rnd(mxp - mnn) / qmax), 0x1p-23f);
  const float zp = fminf(fmaxf(-rintf(D::rnd(mnn / s)), 0.0f), qmax);
  return UxQP{s, D::rnd(1.0f / s), zp};
}

// A float16 group whose scale is below about 2^-16 has an infinite reciprocal: w * inv
// is +inf (code qmax), -inf (code 0) or, for a zero weight, NaN, which the page's
// float-to-uint8 conversion turns into code 0. Tested on the reciprocal's bits, so the
// result does not depend on how the compiler treats NaN.
template <int DT>
__device__ __forceinline__ bool ux_inv_is_inf(float inv) {
  if constexpr (DT == kF16) return __float_as_uint(inv) == 0x7F800000u;
  return false;
}

// q = clamp(rint(r(w * inv)) + zp, 0, qmax). The page rounds the sum to the dtype before
// the clamp: it is an integer below 2^11 or +-inf, so nothing changes.
template <int DT>
__device__ __forceinline__ uint32_t ux_code(float x, const UxQP& q, float qmax) {
  if (ux_inv_is_inf<DT>(q.inv)) return x > 0.0f ? (uint32_t)qmax : 0u;
  const float t = UxDt<DT>::rnd(x * q.inv);
  return (uint32_t)fminf(fmaxf(rintf(t) + q.zp, 0.0f), qmax);
}

// r(r(q - zp) * scale): q - zp is an exact small integer; the product is exact in
// float32 for the 2-byte dtypes (one rounding to the dtype) and one float32 rounding for
// float32 weights.
template <int DT>
__device__ __forceinline__ float ux_value(uint32_t c, float zp, float s) {
  return UxDt<DT>::rnd(((float)c - zp) * s);
}

}  // namespace gwb
