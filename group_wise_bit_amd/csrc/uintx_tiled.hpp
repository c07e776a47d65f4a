// Tiled affine uintx kernels: quantize + pack, unpack + dequantize, fused error, for
// every weight dtype (bfloat16, float16, float32) and group G in {32, 64, 128}.
// Page uintx_quant.py: pack_uintx / unpack_uintx (planar power-of-two shards),
// UIntXQuantizer._quantize_impl and _dequantize_native (arithmetic of uintx_math.hpp).
//
// Planar shards: byte i of the k-bit shard holds codes i, i+L, i+2L, ... (L = that
// shard's byte count), which lie far apart in the matrix. With numel % 8 == 0 the shard
// lengths nest (L_1 = numel/8, L_2 = 2 L_1, L_4 = 4 L_1): the codes at position p of
// the 8 segments j*L_1 + p (j = 0..7) fill byte p of the 1-bit shard, bytes p and
// L_1 + p of the 2-bit shard and bytes m*L_1 + p (m < 4) of the 4-bit shard, and nothing
// else. So a lane that loads the same 8 positions of all 8 segments owns complete output
// bytes and assembles them in registers. With L_1 % G == 0 (numel % 8G == 0) every
// segment starts on a group boundary: a group is G/8 consecutive lanes ("a set") in
// every segment, and a set's 8 groups (one per segment) are shared through LDS.
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"
#include "uintx_layout.hpp"
#include "uintx_math.hpp"

namespace gwb {

// A lane takes 8 consecutive positions p of all 8 segments (elements j*L1 + p), a
// wavefront 512 positions, a block of 4 wavefronts 2048.
constexpr int kLanePos = 8;
constexpr int kWavePos = 64 * kLanePos;
constexpr int kBlockPos = 4 * kWavePos;

inline bool uintx_tiles_fit(int group, int64_t numel) { return numel % (8 * (int64_t)group) == 0; }
inline unsigned uintx_tiles(int64_t numel) { return (unsigned)(((uint64_t)numel / 8 + kBlockPos - 1) / kBlockPos); }

template <bool CONTIG, typename T>
__device__ __forceinline__ T* elem_ptr(T* base, int64_t ld, uint32_t e, FastDiv kdiv) {
  if constexpr (CONTIG) return base + e;
  const uint32_t n = fdiv(e, kdiv);
  return base + (int64_t)n * ld + (e - n * kdiv.d);
}

// Shard bytes are stored non-temporally: the packed tensors are read back much later, if
// at all, and ordinary stores would leave them as dirty lines for the next kernel.
typedef uint32_t ux_u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st8(uint8_t* p, uint32_t lo, uint32_t hi) {
  __builtin_nontemporal_store(ux_u32x2_t{lo, hi}, reinterpret_cast<ux_u32x2_t*>(p));
}
__device__ __forceinline__ uint2 ld8(const uint8_t* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ uint2 ld8_nt(const uint8_t* p) {
  const ux_u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const ux_u32x2_t*>(p));
  return make_uint2(v[0], v[1]);
}

template <typename T>
__device__ __forceinline__ Raw8<T> ux_load_raw8(const T* p) { return load_raw8(p); }

// Min and max of 8 weights. 2-byte dtypes run on order-preserving keys: a word of two
// bf16 or fp16 values read as a float32 orders like its upper value (the lower one only
// extends the mantissa; both formats are sign-magnitude like float32), the word rotated
// by 16 bits like its lower value. ux_key_value recovers the extreme value from its key.
template <int DT>
__device__ __forceinline__ void ux_extremes8(const Raw8<typename UxDt<DT>::T>& r, float& mn, float& mx) {
  float k[8];
  if constexpr (DT == kF32) {
    to_f32(r, k);
  } else {
    const uint32_t w4[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      k[q] = __uint_as_float(w4[q]);
      k[q + 4] = __uint_as_float((w4[q] >> 16) | (w4[q] << 16));
    }
  }
  mn = k[0];
  mx = k[0];
#pragma unroll
  for (int q = 1; q < 8; ++q) {
    mn = fminf(mn, k[q]);
    mx = fmaxf(mx, k[q]);
  }
}
template <int DT>
__device__ __forceinline__ float ux_key_value(float k) {
  if constexpr (DT == kF32) return k;
  else if constexpr (DT == kBF16) return __uint_as_float(__float_as_uint(k) & 0xFFFF0000u);
  else return UxDt<kF16>::value(__float_as_uint(k) >> 16);
}

typedef __bf16 ux_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float ux_f32x2_t __attribute__((ext_vector_type(2)));
// Two float32 rounded to bf16 (RNE, the hardware pair conversion), back as float32.
__device__ __forceinline__ void round_bf16_pair(float& a, float& b) {
  const uint32_t r = __builtin_bit_cast(uint32_t, __builtin_convertvector(ux_f32x2_t{a, b}, ux_bf16x2_t));
  a = __uint_as_float(r << 16);
  b = __uint_as_float(r & 0xFFFF0000u);
}

// Codes of 8 weights as bytes: lo = positions 0..3, hi = 4..7; also the weights x and
// q - zp as floats (what the fused reconstruction sums start from). clamp(rint(t) + zp,
// 0, qmax) is formed as clamp(rint(t), -zp, qmax - zp) + zp: the same integer, with
// q - zp on the way.
template <int DT>
__device__ __forceinline__ void ux_codes8(const Raw8<typename UxDt<DT>::T>& r, float inv, float zp, float qmax,
                                          uint32_t& lo, uint32_t& hi, float* x, float* qz) {
  ux_widen8<DT>(r, x);
  uint32_t w[2] = {0u, 0u};
  if (ux_inv_is_inf<DT>(inv)) {              // float16 only; see ux_inv_is_inf
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float c = x[i] > 0.0f ? qmax : 0.0f;
      qz[i] = c - zp;
      w[i >> 2] |= (uint32_t)c << (8 * (i & 3));
    }
  } else {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = x[i] * inv;   // exact for the 2-byte dtypes (<= 11-bit significands)
    if constexpr (DT == kBF16) {
#pragma unroll
      for (int i = 0; i < 8; i += 2) round_bf16_pair(t[i], t[i + 1]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = UxDt<DT>::rnd(t[i]);
    }
    const float lo_q = -zp, hi_q = qmax - zp;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qz[i] = __builtin_amdgcn_fmed3f(rintf(t[i]), lo_q, hi_q);
      w[i >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(qz[i] + zp, i & 3, w[i >> 2]);
    }
  }
  lo = w[0];
  hi = w[1];
}

// bfloat16 weights: t = x * inv is exact in float32 (two 8-bit significands), and
// bf16(v) as a float32 is one pair conversion of (0, v), whose low half is the zero's.
__device__ __forceinline__ float ux_round_bf16(float v) {
  return __builtin_bit_cast(float, __builtin_convertvector(ux_f32x2_t{0.0f, v}, ux_bf16x2_t));
}
__device__ __forceinline__ void ux_codes8_bf16(const float* x, float inv, float zp, float qmax, uint32_t& lo,
                                               uint32_t& hi, float* qz) {
  uint32_t w[2] = {0u, 0u};
  const float lo_q = -zp, hi_q = qmax - zp;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    qz[i] = __builtin_amdgcn_fmed3f(rintf(ux_round_bf16(x[i] * inv)), lo_q, hi_q);
    w[i >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(qz[i] + zp, i & 3, w[i >> 2]);
  }
  lo = w[0];
  hi = w[1];
}

// ------------------------------------------------------------- tiled quantize
// One block per 2048 positions. Per lane: 8 loads (one per segment) in flight; per
// segment a DPP min/max over the G/8 lanes of a set; each lane of the set then computes
// the qparams of 8/(G/8) of the set's 8 groups (G = 128: lanes 8..15 repeat lanes 0..7)
// and the set exchanges (1/scale, zp) through LDS; codes are assembled into shard bytes
// in registers.
// SNR: also the reconstruction sums of the stored values (the dequantize kernel's
// arithmetic on the codes and scale just written, in its per-thread order), one partial
// pair per block.
template <int NB, int DT, int G, bool CONTIG, bool SNR>
__global__ __launch_bounds__(256) void uintx_quant_tiled(const typename UxDt<DT>::T* __restrict__ W, int64_t ldw,
                                                         FastDiv kdiv, uint32_t L1, Shards sh,
                                                         uint8_t* __restrict__ packed,
                                                         typename UxDt<DT>::T* __restrict__ scales,
                                                         uint8_t* __restrict__ zeros, double* __restrict__ part) {
  using SB = ShardBits<NB>;
  using D = UxDt<DT>;
  constexpr int LG = G / 8;                    // lanes per group
  constexpr int PER = LG >= 8 ? 1 : 8 / LG;    // groups whose qparams one lane computes
  __shared__ typename D::Lds qp_lds[256 / LG * 8];
  __shared__ typename D::Lds qs_lds[SNR ? 256 / LG * 8 : 1];   // (s, zp) as the dequantize kernel reads them
  const float qmax = (float)((1 << NB) - 1);
  const int lane = threadIdx.x & 63;
  const uint32_t p = blockIdx.x * kBlockPos + (threadIdx.x >> 6) * kWavePos + lane * kLanePos;
  const bool active = p < L1;                // whole sets: L1 % G == 0
  typename D::Lds* const set_qp = &qp_lds[(threadIdx.x / LG) * 8];
  Raw8<typename D::T> raw[8];
  bool safe[8];                              // group small enough for float32 squares
  if (active) {
#pragma unroll
    for (int j = 0; j < 8; ++j) raw[j] = ux_load_raw8(elem_ptr<CONTIG>(W, ldw, j * L1 + p, kdiv));
    float mn[8], mx[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float a, b;
      ux_extremes8<DT>(raw[j], a, b);
      mn[j] = lanes_min<LG>(a);
      mx[j] = lanes_max<LG>(b);
      // a 2-byte key orders like, and is below 2^60 exactly when, the weight it holds
      safe[j] = DT == kF16 || fmaxf(fabsf(mn[j]), fabsf(mx[j])) < (DT == kBF16 ? kSafeSqMax64 : kSafeSqMax);
    }
    const int i = lane % LG;
    const uint32_t p0 = p - i * kLanePos;    // the set's first position
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int jj = (i + m * LG) & 7;       // this lane's segment for the qparams
      float mni = mn[0], mxi = mx[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) {
        mni = jj == j ? mn[j] : mni;
        mxi = jj == j ? mx[j] : mxi;
      }
      const UxQP q = ux_qparams<DT>(ux_key_value<DT>(mni), ux_key_value<DT>(mxi), qmax);
      if (LG <= 8 || i < 8) {
        const uint32_t g = (jj * L1 + p0) / G;
        scales[g] = D::word(q.s);
        zeros[g] = (uint8_t)q.zp;
        set_qp[jj] = D::pack(D::word(q.inv), (uint32_t)q.zp);
        if constexpr (SNR) qs_lds[(threadIdx.x / LG) * 8 + jj] = D::pack(D::word(q.s), (uint32_t)q.zp);
      }
    }
  }
  __syncthreads();
  double sw = 0.0, se = 0.0;
  float fa = 0.0f, fb = 0.0f;                // bf16 weights: the lane's float32 sums over its safe segments
  if (active) {
  uint32_t clo[8], chi[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const typename D::Lds w = set_qp[j];
    float x[8], qz[8];
    if constexpr (DT == kBF16) {
      to_f32(raw[j], x);
      ux_codes8_bf16(x, D::lds_value(w), D::lds_zp(w), qmax, clo[j], chi[j], qz);
      // the code words are formed here: left to itself the compiler defers their
      // conversions to the shard packing and keeps all 64 q - zp values live
      asm volatile("" : "+v"(clo[j]), "+v"(chi[j]));
      if constexpr (SNR) {
        const float sc = D::lds_value(qs_lds[(threadIdx.x / LG) * 8 + j]);
        float d[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) d[b] = ux_round_bf16(qz[b] * sc);
        if (safe[j]) acc_err8_f32_bf16_into(raw[j].v, x, d, fa, fb);
        else acc_err8(x, d, sw, se);
      }
      continue;
    }
    ux_codes8<DT>(raw[j], D::lds_value(w), D::lds_zp(w), qmax, clo[j], chi[j], x, qz);
    if constexpr (SNR) {
      // the reconstruction sums of the stored values: r(r(q - zp) * s) as the dequantize
      // kernel forms it (q - zp exact), from the codes just formed
      const float sc = D::lds_value(qs_lds[(threadIdx.x / LG) * 8 + j]);
      float d[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) d[b] = qz[b] * sc;
      if constexpr (DT == kBF16) {
#pragma unroll
        for (int b = 0; b < 8; b += 2) round_bf16_pair(d[b], d[b + 1]);
      } else if constexpr (DT == kF16) {
#pragma unroll
        for (int b = 0; b < 8; ++b) d[b] = D::rnd(d[b]);
      }
      if (!safe[j]) acc_err8(x, d, sw, se);
      else if constexpr (DT == kBF16) acc_err8_f32_bf16(raw[j].v, x, d, sw, se);
      else acc_err8_f32(x, d, sw, se);
    }
  }
  if constexpr (SB::has4) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
      st8(packed + sh.base4 + (int64_t)m * L1 + p, (clo[m] & 0x0F0F0F0Fu) | ((clo[m + 4] & 0x0F0F0F0Fu) << 4),
          (chi[m] & 0x0F0F0F0Fu) | ((chi[m + 4] & 0x0F0F0F0Fu) << 4));
  }
  if constexpr (SB::has2) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        lo |= ((clo[m + 2 * jj] >> SB::off2) & 0x03030303u) << (2 * jj);
        hi |= ((chi[m + 2 * jj] >> SB::off2) & 0x03030303u) << (2 * jj);
      }
      st8(packed + sh.base2 + (int64_t)m * L1 + p, lo, hi);
    }
  }
  if constexpr (SB::has1) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      lo |= ((clo[j] >> SB::off1) & 0x01010101u) << j;
      hi |= ((chi[j] >> SB::off1) & 0x01010101u) << j;
    }
    st8(packed + sh.base1 + p, lo, hi);
  }
  }
  if constexpr (SNR) block_sum2_store<256>(sw + (double)fa, se + (double)fb, part);
}

// ------------------------------------------------------------- tiled dequantize
// SINK kStore writes out (OUT = the weight dtype or kF32), SINK kErr accumulates the
// reconstruction error against W. Each lane loads the scale and zero point of its own
// group in each segment (the eight lanes of a set read the same ones; a wavefront's load
// covers eight consecutive groups), so no lane waits at a barrier for another's loads:
// the shard bytes, the group parameters and the error sink's weights all go out first,
// then each segment's values are formed and stored.
template <int NB, int DT, int G, int SINK, int OUT, bool CONTIG>
__global__ __launch_bounds__(256) void uintx_dequant_tiled(const uint8_t* __restrict__ packed,
                                                           const typename UxDt<DT>::T* __restrict__ scales,
                                                           const uint8_t* __restrict__ zeros, FastDiv kdiv,
                                                           uint32_t L1, Shards sh, void* __restrict__ out,
                                                           int64_t ldo, const typename UxDt<DT>::T* __restrict__ W,
                                                           int64_t ldw, double* __restrict__ part) {
  using SB = ShardBits<NB>;
  using D = UxDt<DT>;
  const int lane = threadIdx.x & 63;
  const uint32_t p = blockIdx.x * kBlockPos + (threadIdx.x >> 6) * kWavePos + lane * kLanePos;
  double sw = 0.0, se = 0.0;
  if (p < L1) {
    uint2 s4[4], s2[2], s1;
    typename D::T sc[8];
    uint32_t zz[8];
    Raw8<typename D::T> wr[8];               // the error sink's weights
    if constexpr (SB::has4) {
#pragma unroll
      for (int m = 0; m < 4; ++m) s4[m] = ld8_nt(packed + sh.base4 + (int64_t)m * L1 + p);
    }
    if constexpr (SB::has2) {
#pragma unroll
      for (int m = 0; m < 2; ++m) s2[m] = ld8_nt(packed + sh.base2 + (int64_t)m * L1 + p);
    }
    if constexpr (SB::has1) s1 = ld8_nt(packed + sh.base1 + p);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t g = (j * L1 + p) / G;   // L1 % G == 0: a lane's 8 positions share a group
      sc[j] = scales[g];
      zz[j] = zeros[g];
    }
    if constexpr (SINK == kErr) {
#pragma unroll
      for (int j = 0; j < 8; ++j) wr[j] = ux_load_raw8(elem_ptr<CONTIG>(W, ldw, j * L1 + p, kdiv));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const typename D::Lds w = D::pack(sc[j], zz[j]);
      const float s = D::lds_value(w), zp = D::lds_zp(w);
      uint32_t c[2] = {0u, 0u};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if constexpr (SB::has4) c[h] |= ((h ? s4[j & 3].y : s4[j & 3].x) >> (4 * (j >> 2))) & 0x0F0F0F0Fu;
        if constexpr (SB::has2) c[h] |= (((h ? s2[j & 1].y : s2[j & 1].x) >> (2 * (j >> 1))) & 0x03030303u) << SB::off2;
        if constexpr (SB::has1) c[h] |= (((h ? s1.y : s1.x) >> j) & 0x01010101u) << SB::off1;
      }
      float d[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) d[b] = ((float)((c[b >> 2] >> (8 * (b & 3))) & 0xFFu) - zp) * s;
      const uint32_t e = j * L1 + p;
      if constexpr (DT == kBF16 && SINK == kStore && OUT == kBF16) {
        // the products are exact: the pair conversion is the one rounding
        U4 v;
        v.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(ux_f32x2_t{d[0], d[1]}, ux_bf16x2_t));
        v.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(ux_f32x2_t{d[2], d[3]}, ux_bf16x2_t));
        v.z = __builtin_bit_cast(uint32_t, __builtin_convertvector(ux_f32x2_t{d[4], d[5]}, ux_bf16x2_t));
        v.w = __builtin_bit_cast(uint32_t, __builtin_convertvector(ux_f32x2_t{d[6], d[7]}, ux_bf16x2_t));
        st16_nt(elem_ptr<CONTIG>((uint16_t*)out, ldo, e, kdiv), v);
        continue;
      }
      if constexpr (DT == kBF16) {
#pragma unroll
        for (int b = 0; b < 8; b += 2) round_bf16_pair(d[b], d[b + 1]);
      } else if constexpr (DT == kF16) {
        if constexpr (SINK == kStore && OUT == kF16) {
          uint32_t hh[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) hh[q] = (uint32_t)D::word(d[2 * q]) | ((uint32_t)D::word(d[2 * q + 1]) << 16);
          st16_nt(elem_ptr<CONTIG>((uint16_t*)out, ldo, e, kdiv), U4{hh[0], hh[1], hh[2], hh[3]});
          continue;
        }
#pragma unroll
        for (int b = 0; b < 8; ++b) d[b] = D::rnd(d[b]);
      }
      if constexpr (SINK == kStore) {
        store8(elem_ptr<CONTIG>((float*)out, ldo, e, kdiv), d);
      } else {
        float x[8];
        ux_widen8<DT>(wr[j], x);
        acc_err8(x, d, sw, se);
      }
    }
  }
  if constexpr (SINK == kErr) block_sum2_store<256>(sw, se, part);
}

// ------------------------------------------------------------- decode GEMV
// y[b, n] = sum_k x[b, k] * w[n, k] with w the weight page uintx_quant.py's forward
// multiplies: r((q - zp) * s) in the weight dtype, converted to the bf16 of the
// activations (one RNE rounding for bf16 weights, the page's two for fp16 and fp32).
// With N % 8 == 0 and K % 512 == 0, position p of segment j is row j * N/8 + p / K,
// column p % K: a lane's 8 positions of the 8 segments share 8 activation columns and feed
// 8 output rows. A wavefront takes CH consecutive 512-position chunks of one row (CH = 4
// when K % 2048 == 0 for up to 4 activation rows, 2 when K % 1024 == 0 for more, else 1:
// the chunks' activations stay in registers, B x CH x 16 bytes per lane, and 8 rows of 4
// chunks left one wavefront per SIMD), so each lane sums 64 * CH weights per row before one transposed
// reduction leaves lane j with row j's sum. The weight pairs meet the activation pairs in
// v_dot2c_f32_bf16; each wavefront writes one partial per row, added over the
// K / (512 CH) wavefronts of a row in order afterwards, or, when one wavefront covers the
// whole row, the row's sum straight into y.
template <int CTRL, int NV>
__device__ __forceinline__ void ux_fold_half(float (&v)[8], bool up) {
#pragma unroll
  for (int i = 0; i < NV / 2; ++i) {
    const float keep = up ? v[i + NV / 2] : v[i], send = up ? v[i] : v[i + NV / 2];
    v[i] = keep + dpp_read<CTRL>(send);
  }
}
// 8 values per lane -> lane l holds the wavefront sum of value (l & 7). The half-mirror
// partner of lane i is 7 - i (differs in bit 2), the quad steps pair bits 1 and 0; then
// the eight 8-lane groups, which hold the same value index, are added.
__device__ __forceinline__ float ux_transposed_sum(float (&v)[8], int lane) {
  ux_fold_half<kDppHalfMirror, 8>(v, lane & 4);
  ux_fold_half<kDppXor2, 4>(v, lane & 2);
  ux_fold_half<kDppXor1, 2>(v, lane & 1);
  float r = v[0];
  r += dpp_read<kDppRor8>(r);
  r += __shfl_xor(r, 16);
  r += __shfl_xor(r, 32);
  return r;
}

// 512-position chunks per wavefront (CH above) for B activation rows.
inline int ux_gemv_chunks(int64_t K, int B) {
  if (B <= 4) return K % 2048 == 0 ? 4 : 1;
  return K % 1024 == 0 ? 2 : 1;
}

// The 4 code bytes of a dword as floats. A code below 16 (NB <= 4) read as an OCP e4m3
// byte is c * 2^-9 exactly (subnormals and the first binade share one spacing), so the
// scaled FP8 conversion at 2^9 gives two per instruction; wider codes convert byte by
// byte.
template <int NB>
__device__ __forceinline__ void ux_code_floats(uint32_t cd, float (&c)[4]) {
  if constexpr (NB <= 4) {
    const ux_f32x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cd, 512.0f, false);
    const ux_f32x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cd, 512.0f, true);
    c[0] = lo[0]; c[1] = lo[1]; c[2] = hi[0]; c[3] = hi[1];
  } else {
    c[0] = (float)(cd & 0xFFu); c[1] = (float)((cd >> 8) & 0xFFu);
    c[2] = (float)((cd >> 16) & 0xFFu); c[3] = (float)(cd >> 24);
  }
}

template <int NB, int DT, int G, int B, int CH>
__global__ __launch_bounds__(256) void uintx_gemv_tiled(const uint8_t* __restrict__ packed,
                                                        const typename UxDt<DT>::T* __restrict__ scales,
                                                        const uint8_t* __restrict__ zeros, FastDiv kdiv, uint32_t L1,
                                                        Shards sh, int N, const uint16_t* __restrict__ x,
                                                        int64_t ldx, int Bn, GemvOut out) {
  using SB = ShardBits<NB>;
  using D = UxDt<DT>;
  constexpr int LG = G / 8;                    // lanes per group
  constexpr int PER = LG >= 8 ? 1 : 8 / LG;    // groups whose parameters one lane loads
  __shared__ typename D::Lds qp_lds[CH][256 / LG * 8];
  const int lane = threadIdx.x & 63;
  const uint32_t p0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * (uint32_t)(kWavePos * CH) + lane * kLanePos;
  const bool active = p0 < L1;               // whole wavefronts: L1 % (512 CH) == 0
  const uint32_t pa = active ? p0 : 0;
  const uint32_t row = fdiv(pa, kdiv), col0 = pa - row * kdiv.d;   // the CH chunks stay in this row
  const int set = threadIdx.x / LG;
  uint2 s4[CH][4], s2[CH][2], s1[CH];
  U4 xv[CH][B];
  if (active) {
    const int i = lane % LG;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint32_t p = p0 + c * kWavePos, ps = p - i * kLanePos;   // ps: the set's first position
#pragma unroll
      for (int m = 0; m < PER; ++m) {
        const int jj = (i + m * LG) & 7;
        const uint32_t g = (jj * L1 + ps) / G;
        const typename D::T sc = scales[g];
        const uint32_t zz = zeros[g];
        if (LG <= 8 || i < 8) qp_lds[c][set * 8 + jj] = D::pack(sc, zz);
      }
      if constexpr (SB::has4) {
#pragma unroll
        for (int m = 0; m < 4; ++m) s4[c][m] = ld8(packed + sh.base4 + (int64_t)m * L1 + p);
      }
      if constexpr (SB::has2) {
#pragma unroll
        for (int m = 0; m < 2; ++m) s2[c][m] = ld8(packed + sh.base2 + (int64_t)m * L1 + p);
      }
      if constexpr (SB::has1) s1[c] = ld8(packed + sh.base1 + p);
#pragma unroll
      for (int b = 0; b < B; ++b) xv[c][b] = ld16(x + (int64_t)min(b, Bn - 1) * ldx + col0 + c * kWavePos);
    }
  }
  __syncthreads();
  if (!active) return;                       // wave-uniform, after the only barrier
  float acc[B][8];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[b][j] = 0.0f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const typename D::Lds* qpo = &qp_lds[c][set * 8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const typename D::Lds w = qpo[j];
      const float s = D::lds_value(w), zp = D::lds_zp(w);
      uint32_t cd[2] = {0u, 0u};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if constexpr (SB::has4) cd[h] |= ((h ? s4[c][j & 3].y : s4[c][j & 3].x) >> (4 * (j >> 2))) & 0x0F0F0F0Fu;
        if constexpr (SB::has2)
          cd[h] |= (((h ? s2[c][j & 1].y : s2[c][j & 1].x) >> (2 * (j >> 1))) & 0x03030303u) << SB::off2;
        if constexpr (SB::has1) cd[h] |= (((h ? s1[c].y : s1[c].x) >> j) & 0x01010101u) << SB::off1;
      }
      float cf[8], d[8];
      ux_code_floats<NB>(cd[0], reinterpret_cast<float(&)[4]>(cf[0]));
      ux_code_floats<NB>(cd[1], reinterpret_cast<float(&)[4]>(cf[4]));
      if constexpr (DT == kF32) {
        // (q - zp) exact, times s: the page's one float32 rounding
#pragma unroll
        for (int q = 0; q < 8; ++q) d[q] = (cf[q] - zp) * s;
      } else {
        // exact in float32 for the 2-byte dtypes: c * s - zp * s as one fma
        const float nzs = -(zp * s);
#pragma unroll
        for (int q = 0; q < 8; ++q) d[q] = __builtin_fmaf(cf[q], s, nzs);
        if constexpr (DT == kF16) {
#pragma unroll
          for (int q = 0; q < 8; ++q) d[q] = D::rnd(d[q]);      // the fp16 weight, then its bf16
        }
      }
      ux_bf16x2_t wp[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) wp[q] = __builtin_convertvector(ux_f32x2_t{d[2 * q], d[2 * q + 1]}, ux_bf16x2_t);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const uint32_t xw[4] = {xv[c][b].x, xv[c][b].y, xv[c][b].z, xv[c][b].w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[b][j] = __builtin_amdgcn_fdot2_f32_bf16(wp[q], __builtin_bit_cast(ux_bf16x2_t, xw[q]), acc[b][j], false);
      }
    }
  }
  const int j = lane & 7;
  const uint32_t chunk = col0 / (kWavePos * CH);
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const float v = ux_transposed_sum(acc[b], lane);
    if (lane < 8 && b < Bn) {
      const int64_t n = (int64_t)j * (N / 8) + row;
      if (out.mode == GemvOut::kPart) out.part[((int64_t)chunk * Bn + b) * N + n] = v;
      else if (out.mode == GemvOut::kF32) static_cast<float*>(out.y)[b * out.ldy + n] = v;
      else static_cast<uint16_t*>(out.y)[b * out.ldy + n] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

// ------------------------------------------------------------------ launchers
// Contiguous rows (ld == K) index elements directly; otherwise through a fast division.
template <int DT, int G, int NB>
void ux_quant_tiled_nb(const void* W, int64_t N, int64_t K, int64_t ldw, void* packed, void* scales, void* zeros,
                       double* part, hipStream_t st) {
  using T = typename UxDt<DT>::T;
  const uint32_t numel = (uint32_t)(N * K);
  if (part)
    hipLaunchKernelGGL((ldw == K ? uintx_quant_tiled<NB, DT, G, true, true> : uintx_quant_tiled<NB, DT, G, false, true>),
                       dim3(uintx_tiles(numel)), dim3(256), 0, st, (const T*)W, ldw, make_fastdiv((uint32_t)K),
                       numel / 8, shards_of(NB, numel), (uint8_t*)packed, (T*)scales, (uint8_t*)zeros, part);
  else
    hipLaunchKernelGGL((ldw == K ? uintx_quant_tiled<NB, DT, G, true, false> : uintx_quant_tiled<NB, DT, G, false, false>),
                       dim3(uintx_tiles(numel)), dim3(256), 0, st, (const T*)W, ldw, make_fastdiv((uint32_t)K),
                       numel / 8, shards_of(NB, numel), (uint8_t*)packed, (T*)scales, (uint8_t*)zeros, part);
}
template <int DT, int G>
void ux_quant_tiled(int nbits, const void* W, int64_t N, int64_t K, int64_t ldw, void* packed, void* scales,
                    void* zeros, double* part, hipStream_t st) {
  switch (nbits) {
    case 2: ux_quant_tiled_nb<DT, G, 2>(W, N, K, ldw, packed, scales, zeros, part, st); break;
    case 3: ux_quant_tiled_nb<DT, G, 3>(W, N, K, ldw, packed, scales, zeros, part, st); break;
    case 4: ux_quant_tiled_nb<DT, G, 4>(W, N, K, ldw, packed, scales, zeros, part, st); break;
    case 5: ux_quant_tiled_nb<DT, G, 5>(W, N, K, ldw, packed, scales, zeros, part, st); break;
    case 6: ux_quant_tiled_nb<DT, G, 6>(W, N, K, ldw, packed, scales, zeros, part, st); break;
    default: ux_quant_tiled_nb<DT, G, 7>(W, N, K, ldw, packed, scales, zeros, part, st); break;
  }
}

template <int DT, int G, int SINK, int OUT, int NB>
void ux_deq_tiled_nb(const void* packed, const void* scales, const void* zeros, int64_t N, int64_t K, void* out,
                     int64_t ldo, const void* W, int64_t ldw, double* part, hipStream_t st) {
  using T = typename UxDt<DT>::T;
  const uint32_t numel = (uint32_t)(N * K);
  const bool contig = SINK == kStore ? ldo == K : ldw == K;
  hipLaunchKernelGGL((contig ? uintx_dequant_tiled<NB, DT, G, SINK, OUT, true>
                             : uintx_dequant_tiled<NB, DT, G, SINK, OUT, false>),
                     dim3(uintx_tiles(numel)), dim3(256), 0, st, (const uint8_t*)packed, (const T*)scales,
                     (const uint8_t*)zeros, make_fastdiv((uint32_t)K), numel / 8, shards_of(NB, numel), out, ldo,
                     (const T*)W, ldw, part);
}
template <int DT, int G, int SINK, int OUT>
void ux_deq_tiled(int nbits, const void* packed, const void* scales, const void* zeros, int64_t N, int64_t K,
                  void* out, int64_t ldo, const void* W, int64_t ldw, double* part, hipStream_t st) {
  switch (nbits) {
    case 2: ux_deq_tiled_nb<DT, G, SINK, OUT, 2>(packed, scales, zeros, N, K, out, ldo, W, ldw, part, st); break;
    case 3: ux_deq_tiled_nb<DT, G, SINK, OUT, 3>(packed, scales, zeros, N, K, out, ldo, W, ldw, part, st); break;
    case 4: ux_deq_tiled_nb<DT, G, SINK, OUT, 4>(packed, scales, zeros, N, K, out, ldo, W, ldw, part, st); break;
    case 5: ux_deq_tiled_nb<DT, G, SINK, OUT, 5>(packed, scales, zeros, N, K, out, ldo, W, ldw, part, st); break;
    case 6: ux_deq_tiled_nb<DT, G, SINK, OUT, 6>(packed, scales, zeros, N, K, out, ldo, W, ldw, part, st); break;
    default: ux_deq_tiled_nb<DT, G, SINK, OUT, 7>(packed, scales, zeros, N, K, out, ldo, W, ldw, part, st); break;
  }
}

// Every tiled entry of one (dtype, group): quantize, dequantize to the weight dtype or
// float32, and the error sink. Instantiated per (dtype, group) in its own source file.
template <int DT, int G>
void ux_tiled_quant_entry(int nbits, const void* W, int64_t N, int64_t K, int64_t ldw, void* packed, void* scales,
                          void* zeros, double* part, hipStream_t st) {
  ux_quant_tiled<DT, G>(nbits, W, N, K, ldw, packed, scales, zeros, part, st);
}
template <int DT, int G>
void ux_tiled_dequant_entry(int nbits, const void* packed, const void* scales, const void* zeros, int64_t N,
                            int64_t K, void* out, int32_t out_dtype, int64_t ldo, hipStream_t st) {
  if (out_dtype == kF32)
    ux_deq_tiled<DT, G, kStore, kF32>(nbits, packed, scales, zeros, N, K, out, ldo, nullptr, 0, nullptr, st);
  else
    ux_deq_tiled<DT, G, kStore, DT>(nbits, packed, scales, zeros, N, K, out, ldo, nullptr, 0, nullptr, st);
}
template <int DT, int G>
void ux_tiled_err_entry(int nbits, const void* W, int64_t N, int64_t K, int64_t ldw, const void* packed,
                        const void* scales, const void* zeros, double* part, hipStream_t st) {
  ux_deq_tiled<DT, G, kErr, kF32>(nbits, packed, scales, zeros, N, K, nullptr, 0, W, ldw, part, st);
}

template <int DT, int G, int NB, int B, int CH>
void ux_gemv_launch(int Bn, const void* packed, const void* scales, const void* zeros, int64_t N, int64_t K,
                    const void* x, int64_t ldx, GemvOut out, hipStream_t st) {
  const uint32_t numel = (uint32_t)(N * K);
  const unsigned blocks = (unsigned)(((uint64_t)numel / 8 / (kWavePos * CH) + 3) / 4);
  hipLaunchKernelGGL((uintx_gemv_tiled<NB, DT, G, B, CH>), dim3(blocks), dim3(256), 0, st, (const uint8_t*)packed,
                     (const typename UxDt<DT>::T*)scales, (const uint8_t*)zeros, make_fastdiv((uint32_t)K),
                     numel / 8, shards_of(NB, numel), (int)N, (const uint16_t*)x, ldx, Bn, out);
}
template <int DT, int G, int NB, int CH>
void ux_gemv_b(int B, const void* packed, const void* scales, const void* zeros, int64_t N, int64_t K, const void* x,
               int64_t ldx, GemvOut out, hipStream_t st) {
  if (B == 1) ux_gemv_launch<DT, G, NB, 1, CH>(B, packed, scales, zeros, N, K, x, ldx, out, st);
  else if (B == 2) ux_gemv_launch<DT, G, NB, 2, CH>(B, packed, scales, zeros, N, K, x, ldx, out, st);
  else if (B <= 4) ux_gemv_launch<DT, G, NB, 4, CH>(B, packed, scales, zeros, N, K, x, ldx, out, st);
  else ux_gemv_launch<DT, G, NB, 8, CH>(B, packed, scales, zeros, N, K, x, ldx, out, st);
}
template <int DT, int G, int NB>
void ux_gemv_nb(int B, const void* packed, const void* scales, const void* zeros, int64_t N, int64_t K, const void* x,
                int64_t ldx, GemvOut out, hipStream_t st) {
  const int ch = ux_gemv_chunks(K, B);
  if (ch == 4 && B == 1) ux_gemv_launch<DT, G, NB, 1, 4>(B, packed, scales, zeros, N, K, x, ldx, out, st);
  else if (ch == 4 && B == 2) ux_gemv_launch<DT, G, NB, 2, 4>(B, packed, scales, zeros, N, K, x, ldx, out, st);
  else if (ch == 4) ux_gemv_launch<DT, G, NB, 4, 4>(B, packed, scales, zeros, N, K, x, ldx, out, st);
  else if (ch == 2) ux_gemv_launch<DT, G, NB, 8, 2>(B, packed, scales, zeros, N, K, x, ldx, out, st);
  else ux_gemv_b<DT, G, NB, 1>(B, packed, scales, zeros, N, K, x, ldx, out, st);
}
// The decode GEMV of one (dtype, group): N % 8 == 0, K % 512 == 0, B <= 8.
template <int DT, int G>
void ux_tiled_gemv_entry(int nbits, int B, const void* packed, const void* scales, const void* zeros, int64_t N,
                         int64_t K, const void* x, int64_t ldx, GemvOut out, hipStream_t st) {
  switch (nbits) {
    case 2: ux_gemv_nb<DT, G, 2>(B, packed, scales, zeros, N, K, x, ldx, out, st); break;
    case 3: ux_gemv_nb<DT, G, 3>(B, packed, scales, zeros, N, K, x, ldx, out, st); break;
    case 4: ux_gemv_nb<DT, G, 4>(B, packed, scales, zeros, N, K, x, ldx, out, st); break;
    case 5: ux_gemv_nb<DT, G, 5>(B, packed, scales, zeros, N, K, x, ldx, out, st); break;
    case 6: ux_gemv_nb<DT, G, 6>(B, packed, scales, zeros, N, K, x, ldx, out, st); break;
    default: ux_gemv_nb<DT, G, 7>(B, packed, scales, zeros, N, K, x, ldx, out, st); break;
  }
}

}  // namespace gwb
