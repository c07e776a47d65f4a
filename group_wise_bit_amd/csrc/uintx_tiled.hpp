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

__device__ __forceinline__ void st8(uint8_t* p, uint32_t lo, uint32_t hi) {
  *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
}
__device__ __forceinline__ uint2 ld8(const uint8_t* p) { return *reinterpret_cast<const uint2*>(p); }

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

// Codes of 8 weights as bytes: lo = positions 0..3, hi = 4..7.
template <int DT>
__device__ __forceinline__ void ux_codes8(const Raw8<typename UxDt<DT>::T>& r, float inv, float zp, float qmax,
                                          uint32_t& lo, uint32_t& hi) {
  float x[8];
  ux_widen8<DT>(r, x);
  uint32_t w[2] = {0u, 0u};
  if (ux_inv_is_inf<DT>(inv)) {              // float16 only; see ux_inv_is_inf
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i >> 2] |= (x[i] > 0.0f ? (uint32_t)qmax : 0u) << (8 * (i & 3));
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
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float c = __builtin_amdgcn_fmed3f(rintf(t[i]) + zp, 0.0f, qmax);
      w[i >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(c, i & 3, w[i >> 2]);
    }
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
template <int NB, int DT, int G, bool CONTIG>
__global__ __launch_bounds__(256) void uintx_quant_tiled(const typename UxDt<DT>::T* __restrict__ W, int64_t ldw,
                                                         FastDiv kdiv, uint32_t L1, Shards sh,
                                                         uint8_t* __restrict__ packed,
                                                         typename UxDt<DT>::T* __restrict__ scales,
                                                         uint8_t* __restrict__ zeros) {
  using SB = ShardBits<NB>;
  using D = UxDt<DT>;
  constexpr int LG = G / 8;                    // lanes per group
  constexpr int PER = LG >= 8 ? 1 : 8 / LG;    // groups whose qparams one lane computes
  __shared__ typename D::Lds qp_lds[256 / LG * 8];
  const float qmax = (float)((1 << NB) - 1);
  const int lane = threadIdx.x & 63;
  const uint32_t p = blockIdx.x * kBlockPos + (threadIdx.x >> 6) * kWavePos + lane * kLanePos;
  const bool active = p < L1;                // whole sets: L1 % G == 0
  typename D::Lds* const set_qp = &qp_lds[(threadIdx.x / LG) * 8];
  Raw8<typename D::T> raw[8];
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
      }
    }
  }
  __syncthreads();
  if (!active) return;
  uint32_t clo[8], chi[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const typename D::Lds w = set_qp[j];
    ux_codes8<DT>(raw[j], D::lds_value(w), D::lds_zp(w), qmax, clo[j], chi[j]);
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

// ------------------------------------------------------------- tiled dequantize
// SINK kStore writes out (OUT = the weight dtype or kF32), SINK kErr accumulates the
// reconstruction error against W. The set's scales and zero points go first: the LDS
// exchange waits only for them, while the shard bytes and the weights stay in flight
// across the barrier.
template <int NB, int DT, int G, int SINK, int OUT, bool CONTIG>
__global__ __launch_bounds__(256) void uintx_dequant_tiled(const uint8_t* __restrict__ packed,
                                                           const typename UxDt<DT>::T* __restrict__ scales,
                                                           const uint8_t* __restrict__ zeros, FastDiv kdiv,
                                                           uint32_t L1, Shards sh, void* __restrict__ out,
                                                           int64_t ldo, const typename UxDt<DT>::T* __restrict__ W,
                                                           int64_t ldw, double* __restrict__ part) {
  using SB = ShardBits<NB>;
  using D = UxDt<DT>;
  constexpr int LG = G / 8;
  constexpr int PER = LG >= 8 ? 1 : 8 / LG;
  __shared__ typename D::Lds qp_lds[256 / LG * 8];
  const int lane = threadIdx.x & 63;
  const uint32_t p = blockIdx.x * kBlockPos + (threadIdx.x >> 6) * kWavePos + lane * kLanePos;
  const bool active = p < L1;
  typename D::Lds* const set_qp = &qp_lds[(threadIdx.x / LG) * 8];
  uint2 s4[4], s2[2], s1;
  Raw8<typename D::T> wr[8];                 // the error sink's weights
  if (active) {
    const int i = lane % LG;
    const uint32_t p0 = p - i * kLanePos;
    typename D::T sc[PER];
    uint32_t zz[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const uint32_t g = (((i + m * LG) & 7) * L1 + p0) / G;
      sc[m] = scales[g];
      zz[m] = zeros[g];
    }
    if constexpr (SB::has4) {
#pragma unroll
      for (int m = 0; m < 4; ++m) s4[m] = ld8(packed + sh.base4 + (int64_t)m * L1 + p);
    }
    if constexpr (SB::has2) {
#pragma unroll
      for (int m = 0; m < 2; ++m) s2[m] = ld8(packed + sh.base2 + (int64_t)m * L1 + p);
    }
    if constexpr (SB::has1) s1 = ld8(packed + sh.base1 + p);
    if constexpr (SINK == kErr) {
#pragma unroll
      for (int j = 0; j < 8; ++j) wr[j] = ux_load_raw8(elem_ptr<CONTIG>(W, ldw, j * L1 + p, kdiv));
    }
#pragma unroll
    for (int m = 0; m < PER; ++m)
      if (LG <= 8 || i < 8) set_qp[(i + m * LG) & 7] = D::pack(sc[m], zz[m]);
  }
  __syncthreads();
  double sw = 0.0, se = 0.0;
  if (active) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const typename D::Lds w = set_qp[j];
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
          uint32_t h[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) h[q] = (uint32_t)D::word(d[2 * q]) | ((uint32_t)D::word(d[2 * q + 1]) << 16);
          st16_nt(elem_ptr<CONTIG>((uint16_t*)out, ldo, e, kdiv), U4{h[0], h[1], h[2], h[3]});
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

// ------------------------------------------------------------------ launchers
// Contiguous rows (ld == K) index elements directly; otherwise through a fast division.
template <int DT, int G, int NB>
void ux_quant_tiled_nb(const void* W, int64_t N, int64_t K, int64_t ldw, void* packed, void* scales, void* zeros,
                       hipStream_t st) {
  using T = typename UxDt<DT>::T;
  const uint32_t numel = (uint32_t)(N * K);
  hipLaunchKernelGGL((ldw == K ? uintx_quant_tiled<NB, DT, G, true> : uintx_quant_tiled<NB, DT, G, false>),
                     dim3(uintx_tiles(numel)), dim3(256), 0, st, (const T*)W, ldw, make_fastdiv((uint32_t)K),
                     numel / 8, shards_of(NB, numel), (uint8_t*)packed, (T*)scales, (uint8_t*)zeros);
}
template <int DT, int G>
void ux_quant_tiled(int nbits, const void* W, int64_t N, int64_t K, int64_t ldw, void* packed, void* scales,
                    void* zeros, hipStream_t st) {
  switch (nbits) {
    case 2: ux_quant_tiled_nb<DT, G, 2>(W, N, K, ldw, packed, scales, zeros, st); break;
    case 3: ux_quant_tiled_nb<DT, G, 3>(W, N, K, ldw, packed, scales, zeros, st); break;
    case 4: ux_quant_tiled_nb<DT, G, 4>(W, N, K, ldw, packed, scales, zeros, st); break;
    case 5: ux_quant_tiled_nb<DT, G, 5>(W, N, K, ldw, packed, scales, zeros, st); break;
    case 6: ux_quant_tiled_nb<DT, G, 6>(W, N, K, ldw, packed, scales, zeros, st); break;
    default: ux_quant_tiled_nb<DT, G, 7>(W, N, K, ldw, packed, scales, zeros, st); break;
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
                          void* zeros, hipStream_t st) {
  ux_quant_tiled<DT, G>(nbits, W, N, K, ldw, packed, scales, zeros, st);
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

}  // namespace gwb
