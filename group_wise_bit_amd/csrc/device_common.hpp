// Device helpers shared by the gfx950 kernels: DPP group reductions within a
// 64-wide wavefront, bfloat16 bit conversions, 32-bit fast division and the
// workspace reduction used by the fused error kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gwb {

// ---------------------------------------------------------------- DPP controls
// quad_perm(1,0,3,2): lane i reads lane i^1;  quad_perm(2,3,0,1): lane i reads i^2.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
// row_half_mirror: within each 8 lanes, lane i reads 7-i (after the quad steps every
// quad is uniform, so this joins the two quads of an 8-lane half-row).
constexpr int kDppHalfMirror = 0x141;
// row_mirror: within each 16-lane row, lane i reads 15-i (joins the two half-rows).
constexpr int kDppMirror = 0x140;
// row_ror:8: within each 16-lane row, lane i reads lane (i + 8) % 16.
constexpr int kDppRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ float dpp_read(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_read_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}

// Max / min over LANES consecutive, aligned lanes (LANES in {1, 2, 4, 8, 16}); every
// lane of the set ends with the result. All sources lie inside the set.
template <int LANES>
__device__ __forceinline__ float lanes_max(float x) {
  if constexpr (LANES >= 2) x = fmaxf(x, dpp_read<kDppXor1>(x));
  if constexpr (LANES >= 4) x = fmaxf(x, dpp_read<kDppXor2>(x));
  if constexpr (LANES >= 8) x = fmaxf(x, dpp_read<kDppHalfMirror>(x));
  if constexpr (LANES >= 16) x = fmaxf(x, dpp_read<kDppMirror>(x));
  static_assert(LANES <= 16, "groups wider than a DPP row are not used");
  return x;
}
template <int LANES>
__device__ __forceinline__ float lanes_min(float x) {
  if constexpr (LANES >= 2) x = fminf(x, dpp_read<kDppXor1>(x));
  if constexpr (LANES >= 4) x = fminf(x, dpp_read<kDppXor2>(x));
  if constexpr (LANES >= 8) x = fminf(x, dpp_read<kDppHalfMirror>(x));
  if constexpr (LANES >= 16) x = fminf(x, dpp_read<kDppMirror>(x));
  return x;
}

// ---------------------------------------------------------------- bfloat16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// float32 -> bfloat16 bits, round to nearest, ties to even (finite and inf inputs;
// subnormals round like any other value since bfloat16 shares float32's exponent).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (b >> 16) | 0x40u;  // NaN stays NaN
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}
// float32 rounded to the nearest bfloat16 value, kept as a float32.
__device__ __forceinline__ float round_bf16(float f) {
  return __uint_as_float(f32_to_bf16_rne(f) << 16);
}

// ---------------------------------------------------------------- fast division
// q = n / d for 0 <= n < 2^31 via q = (umulhi(n, m) + n) >> s (Granlund-Montgomery).
struct FastDiv {
  uint32_t d, m, s;
};
inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f{d, 0u, 0u};
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.s = s;
  f.m = (uint32_t)((((1ull << s) - d) << 32) / d + 1);
  return f;
}
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
  return (uint32_t)(((uint64_t)__umulhi(n, f.m) + n) >> f.s);
}

// ---------------------------------------------------------------- loads
struct alignas(16) U4 { uint32_t x, y, z, w; };

__device__ __forceinline__ U4 ld16(const void* p) {
  return *reinterpret_cast<const U4*>(p);
}
__device__ __forceinline__ void st16(void* p, U4 v) { *reinterpret_cast<U4*>(p) = v; }

// Rows [ks, kend) of the bf16 activations x (Bn rows, row stride ldx) into LDS rows of
// pitch xp elements, by a 256-thread block: each thread issues up to eight 16-byte loads
// before it writes any (a load-then-write loop waits a full round trip per load).
__device__ __forceinline__ void stage_rows(uint16_t* xs, int xp, const uint16_t* __restrict__ x, int64_t ldx, int Bn,
                                           int ks, int kend) {
  const int cpr = (kend - ks) / 8, total = Bn * cpr;
  for (int v0 = (int)threadIdx.x; v0 < total; v0 += 8 * 256) {
    U4 tmp[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int v = min(v0 + 256 * u, total - 1), b = v / cpr, c = v - b * cpr;   // past the end: re-read the last
      tmp[u] = ld16(x + (int64_t)b * ldx + ks + 8 * c);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int v = v0 + 256 * u, b = v / cpr, c = v - b * cpr;
      if (v < total) *reinterpret_cast<U4*>(xs + b * xp + 8 * c) = tmp[u];
    }
  }
}

// Non-temporal (streaming) variants: data read or written exactly once.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ U4 ld16_nt(const void* p) {
  u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return U4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ void st16_nt(void* p, U4 v) {
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ uint32_t ld4_nt(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st4_nt(uint32_t* p, uint32_t v) { __builtin_nontemporal_store(v, p); }

// Raw weights of one 8-element unit: one 16-byte load of bf16, two of float32.
template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> { U4 v; };
template <> struct Raw8<float> { U4 a, b; };
__device__ __forceinline__ Raw8<uint16_t> load_raw8(const uint16_t* p) { return Raw8<uint16_t>{ld16_nt(p)}; }
__device__ __forceinline__ Raw8<float> load_raw8(const float* p) { return Raw8<float>{ld16_nt(p), ld16_nt(p + 4)}; }
__device__ __forceinline__ void to_f32(const Raw8<uint16_t>& r, float* x) {
  x[0] = __uint_as_float(r.v.x << 16); x[1] = __uint_as_float(r.v.x & 0xFFFF0000u);
  x[2] = __uint_as_float(r.v.y << 16); x[3] = __uint_as_float(r.v.y & 0xFFFF0000u);
  x[4] = __uint_as_float(r.v.z << 16); x[5] = __uint_as_float(r.v.z & 0xFFFF0000u);
  x[6] = __uint_as_float(r.v.w << 16); x[7] = __uint_as_float(r.v.w & 0xFFFF0000u);
}
__device__ __forceinline__ void to_f32(const Raw8<float>& r, float* x) {
  x[0] = __uint_as_float(r.a.x); x[1] = __uint_as_float(r.a.y); x[2] = __uint_as_float(r.a.z); x[3] = __uint_as_float(r.a.w);
  x[4] = __uint_as_float(r.b.x); x[5] = __uint_as_float(r.b.y); x[6] = __uint_as_float(r.b.z); x[7] = __uint_as_float(r.b.w);
}

// Load 8 consecutive weights (16-byte aligned start) as float32.
__device__ __forceinline__ void load8(const uint16_t* p, float* x) {
  U4 v = ld16(p);
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}
__device__ __forceinline__ void load8(const float* p, float* x) {
  U4 a = ld16(p), b = ld16(p + 4);
  x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
  x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
  x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y);
  x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
}

// Two float32 -> packed bf16 pair (a in the low half), round to nearest even: the
// hardware pair conversion (v_cvt_pk_bf16_f32; float32 denormals are kept).
typedef __bf16 dc_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float dc_f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(dc_f32x2_t{a, b}, dc_bf16x2_t));
}

// Store 8 float32 values as bf16 (RNE; one 16-byte non-temporal store) or as float32.
// The float32 run is 32 bytes, two store instructions that each cover half of every
// line the wavefront writes: ordinary stores let L2 merge the halves before HBM
// (non-temporal ones measured 1.5x slower).
__device__ __forceinline__ void store8(uint16_t* p, const float* d) {
  st16_nt(p, U4{pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]), pack_bf16x2(d[4], d[5]), pack_bf16x2(d[6], d[7])});
}
__device__ __forceinline__ void store8(float* p, const float* d) {
  st16(p, U4{__float_as_uint(d[0]), __float_as_uint(d[1]), __float_as_uint(d[2]), __float_as_uint(d[3])});
  st16(p + 4, U4{__float_as_uint(d[4]), __float_as_uint(d[5]), __float_as_uint(d[6]), __float_as_uint(d[7])});
}

// Accumulate sum w^2 and sum (w - d)^2 of 8 elements (w - d a float32 subtraction,
// squares and sums in float64, where the squares are exact).
__device__ __forceinline__ void acc_err8(const float* x, const float* d, double& sw, double& se) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double xd = (double)x[i];
    const double ed = (double)(x[i] - d[i]);
    sw = fma(xd, xd, sw);
    se = fma(ed, ed, se);
  }
}

// Sums of w^2 and (w - d)^2 over the 8 weights of a unit for the fused quantize+SNR
// kernels: the squares and the seven additions of each sum in float32 (one rounding
// each, fused multiply-adds), then one float64 addition per sum and unit, where acc_err8
// squares and adds every weight in float64. The terms are non-negative, so each unit's
// float32 sums are within 8 * 2^-24 of their exact values, relative; values below
// float32's normal range add at most 2^-126 absolute per operation. No float32 value
// overflows while |w| < 2^60 and |w - d| < 2^62: callers take acc_err8 for any group
// whose largest magnitude reaches 2^60 (kSafeSqMax).
constexpr float kSafeSqMax = 0x1p60f;
__device__ __forceinline__ void acc_err8_f32(const float* x, const float* d, double& sw, double& se) {
  float a = x[0] * x[0];
  float e = x[0] - d[0];
  float b = e * e;
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    a = __builtin_fmaf(x[i], x[i], a);
    e = x[i] - d[i];
    b = __builtin_fmaf(e, e, b);
  }
  sw += (double)a;
  se += (double)b;
}

// The same for bf16 weights given as their raw words: each pair's squares in one
// v_dot2_f32_bf16 (both products exact, one accumulation).
__device__ __forceinline__ void acc_err8_f32_bf16(U4 v, const float* x, const float* d, double& sw, double& se) {
  float a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(dc_bf16x2_t, v.x), __builtin_bit_cast(dc_bf16x2_t, v.x),
                                            0.0f, false);
  a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(dc_bf16x2_t, v.y), __builtin_bit_cast(dc_bf16x2_t, v.y), a, false);
  a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(dc_bf16x2_t, v.z), __builtin_bit_cast(dc_bf16x2_t, v.z), a, false);
  a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(dc_bf16x2_t, v.w), __builtin_bit_cast(dc_bf16x2_t, v.w), a, false);
  float e = x[0] - d[0];
  float b = e * e;
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    e = x[i] - d[i];
    b = __builtin_fmaf(e, e, b);
  }
  sw += (double)a;
  se += (double)b;
}

// The bf16 sums of up to 8 units (64 weights) kept in one lane's float32 running sums,
// fa and fb, before one float64 addition each at the end of the lane's work: every step
// is one float32 rounding of a sum of non-negative terms, so for n terms the result is
// within (n + 2) * 2^-24 of the exact sum, relative (66 * 2^-24, about 4e-6 or 2e-5 dB,
// for 64). No float32 value overflows while |w| < 2^56 and |w - d| < 2^58: callers take
// acc_err8 for any group whose largest magnitude reaches 2^56 (kSafeSqMax64).
constexpr float kSafeSqMax64 = 0x1p56f;
__device__ __forceinline__ void acc_err8_f32_bf16_into(U4 v, const float* x, const float* d, float& fa, float& fb) {
  fa = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(dc_bf16x2_t, v.x), __builtin_bit_cast(dc_bf16x2_t, v.x), fa, false);
  fa = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(dc_bf16x2_t, v.y), __builtin_bit_cast(dc_bf16x2_t, v.y), fa, false);
  fa = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(dc_bf16x2_t, v.z), __builtin_bit_cast(dc_bf16x2_t, v.z), fa, false);
  fa = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(dc_bf16x2_t, v.w), __builtin_bit_cast(dc_bf16x2_t, v.w), fa, false);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float e = x[i] - d[i];
    fb = __builtin_fmaf(e, e, fb);
  }
}

// ---------------------------------------------------------------- error sums
// Sum of a double over the 64 lanes of a wavefront, the same value in every lane: DPP
// steps inside each 16-lane row (quad xor 1 and 2, half mirror, mirror: after each step
// the lanes being joined hold equal values, and a + b == b + a, so every lane of a row
// ends with the same sum), then the four row sums read from lanes 0, 16, 32 and 48 and
// added in that order. Fixed order: deterministic. No LDS traffic (a butterfly of
// cross-lane shuffles costs an LDS round trip per step).
template <int CTRL>
__device__ __forceinline__ double dpp_read_f64(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, true);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double readlane_f64(double x, int lane) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_read_f64<kDppXor1>(v);
  v += dpp_read_f64<kDppXor2>(v);
  v += dpp_read_f64<kDppHalfMirror>(v);
  v += dpp_read_f64<kDppMirror>(v);
  return ((readlane_f64(v, 0) + readlane_f64(v, 16)) + readlane_f64(v, 32)) + readlane_f64(v, 48);
}

// Block-wide sum of two doubles; thread 0 writes them to part[2*blockIdx.x]. Each
// wavefront's sum (wave_sum_f64), then thread 0 adds the wavefront sums in order, so
// the result is deterministic for a given launch shape.
template <int THREADS>
__device__ __forceinline__ void block_sum2_store(double a, double b, double* part) {
  static_assert(THREADS % 64 == 0 && THREADS <= 1024, "whole wavefronts");
  __shared__ double sa[THREADS / 64], sb[THREADS / 64];
  a = wave_sum_f64(a);
  b = wave_sum_f64(b);
  if ((threadIdx.x & 63) == 0) {
    sa[threadIdx.x >> 6] = a;
    sb[threadIdx.x >> 6] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double ta = sa[0], tb = sb[0];
#pragma unroll
    for (int i = 1; i < THREADS / 64; ++i) {
      ta += sa[i];
      tb += sb[i];
    }
    part[2 * blockIdx.x] = ta;
    part[2 * blockIdx.x + 1] = tb;
  }
}

}  // namespace gwb
