// Affine uint2..uint7 (torchao-style, preserve_zero, bfloat16 arithmetic) quantize+
// pack into planar power-of-two shards, unpack+dequantize, fused reconstruction error.
// Page uintx_quant.py: _pack_shard, pack_uintx, unpack_uintx,
// UIntXQuantizer._quantize_impl and _dequantize_native. Group 64 along K.
//
// Planar shards: byte i of the k-bit shard holds codes i, i+L, i+2L, ... (L = that
// shard's byte count), which lie far apart in the matrix. With numel % 512 == 0 the
// shard lengths nest (L_1 = numel/8, L_2 = 2 L_1, L_4 = 4 L_1): the codes at position
// p of the 8 segments j*L_1 + p (j = 0..7) fill byte p of the 1-bit shard, bytes
// p and L_1 + p of the 2-bit shard and bytes m*L_1 + p (m < 4) of the 4-bit shard, and
// nothing else. So a lane that loads the same 8 positions of all 8 segments owns
// complete output bytes and assembles them in registers. Segments start on group
// boundaries, so each group's qparams stay within the 8 lanes that hold it.
// Other sizes take a two-pass path: codes to workspace, then one thread per byte.
#include "device_common.hpp"
#include "kernels.hpp"
#include "uintx_layout.hpp"

namespace gwb {

// Tiled path geometry: a lane takes 8 consecutive positions p of all 8 segments
// (elements j*L1 + p), a wavefront 512 positions, a block of 4 wavefronts 2048.
constexpr int kLanePos = 8;
constexpr int kWavePos = 64 * kLanePos;
constexpr int kBlockPos = 4 * kWavePos;

// Group qparams from the group's min and max (every op a float32 op rounded to bf16):
// mn = min(min, 0), mx = max(max, 0); scale = bf(bf(mx - mn) / qmax), at least 2^-23;
// zp = clamp(-rint(bf(mn / scale)), 0, qmax); inv = bf(1 / scale).
struct QP { float s, inv, zp; };
__device__ __forceinline__ QP uintx_qparams(float mn, float mx, float qmax) {
  float mnn = fminf(mn, 0.0f), mxp = fmaxf(mx, 0.0f);
  float s = round_bf16(round_bf16(mxp - mnn) / qmax);
  s = fmaxf(s, 0x1p-23f);
  float zp = fminf(fmaxf(-rintf(round_bf16(mnn / s)), 0.0f), qmax);
  return QP{s, round_bf16(1.0f / s), zp};
}
// q = clamp(rint(bf(w * inv)) + zp, 0, qmax). The page rounds the sum to bf16 before
// the clamp; rounding is monotonic and 0 and qmax are bf16 integers, so the clamped
// result is the same.
__device__ __forceinline__ uint32_t uintx_code(float x, const QP& q, float qmax) {
  float t = round_bf16(x * q.inv);
  return (uint32_t)fminf(fmaxf(rintf(t) + q.zp, 0.0f), qmax);
}
// bf(bf(q - zp) * scale): q - zp is an exact small integer, the product is exact in
// float32, so this is one rounding.
__device__ __forceinline__ float uintx_value(uint32_t c, float zp, float s) {
  return round_bf16(((float)c - zp) * s);
}

typedef __bf16 ux_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float ux_f32x2_t __attribute__((ext_vector_type(2)));
// Two float32 rounded to bf16 (RNE, the hardware pair conversion), back as float32.
__device__ __forceinline__ void round_bf16_pair(float& a, float& b) {
  const uint32_t r = __builtin_bit_cast(uint32_t, __builtin_convertvector(ux_f32x2_t{a, b}, ux_bf16x2_t));
  a = __uint_as_float(r << 16);
  b = __uint_as_float(r & 0xFFFF0000u);
}

// Codes of 8 bf16 weights (one 16-byte load) as bytes: lo = positions 0..3, hi = 4..7.
__device__ __forceinline__ void codes8(U4 v, float inv, float zp, float qmax, uint32_t& lo, uint32_t& hi) {
  float x[8];
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] *= inv;                      // exact: 8-bit x 8-bit significands
#pragma unroll
  for (int i = 0; i < 8; i += 2) round_bf16_pair(x[i], x[i + 1]);
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float c = __builtin_amdgcn_fmed3f(rintf(x[i]) + zp, 0.0f, qmax);
    w[i >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(c, i & 3, w[i >> 2]);
  }
  lo = w[0];
  hi = w[1];
}

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

// ------------------------------------------------------------- tiled quantize
// One block per 2048 positions. Per lane: 8 loads (one per segment) in flight; per
// segment a DPP min/max over the 8 lanes that share each 64-weight group; each of
// those lanes then computes the qparams of one segment's group (lane & 7) and they
// exchange (1/scale, zp) through LDS; codes are assembled into shard bytes in registers.
template <int NB, bool CONTIG>
__global__ __launch_bounds__(256) void uintx_quant_tiled(const uint16_t* __restrict__ W, int64_t ldw, FastDiv kdiv,
                                                         uint32_t L1, Shards sh, uint8_t* __restrict__ packed,
                                                         uint16_t* __restrict__ scales,
                                                         uint8_t* __restrict__ zeros) {
  using SB = ShardBits<NB>;
  __shared__ uint32_t qp_lds[256];
  const float qmax = (float)((1 << NB) - 1);
  const int lane = threadIdx.x & 63;
  const uint32_t p = blockIdx.x * kBlockPos + (threadIdx.x >> 6) * kWavePos + lane * kLanePos;
  const bool active = p < L1;                // whole groups of 8 lanes: L1 % 64 == 0
  U4 raw[8];
  if (active) {
#pragma unroll
    for (int j = 0; j < 8; ++j) raw[j] = ld16_nt(elem_ptr<CONTIG>(W, ldw, j * L1 + p, kdiv));
    // Extremes on order-preserving keys: a word of two bf16 read as a float32 orders
    // like its upper weight (the lower one only extends the mantissa), the word rotated
    // by 16 bits like its lower weight; clearing the low 16 bits of the extreme key
    // gives that weight exactly.
    float mn[8], mx[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w4[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
      float k[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        k[q] = __uint_as_float(w4[q]);
        k[q + 4] = __uint_as_float((w4[q] >> 16) | (w4[q] << 16));
      }
      float a = k[0], b = k[0];
#pragma unroll
      for (int q = 1; q < 8; ++q) {
        a = fminf(a, k[q]);
        b = fmaxf(b, k[q]);
      }
      mn[j] = lanes_min<8>(a);
      mx[j] = lanes_max<8>(b);
    }
    const int i = lane & 7;                  // this lane's segment for the qparams
    float mni = mn[0], mxi = mx[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      mni = i == j ? mn[j] : mni;
      mxi = i == j ? mx[j] : mxi;
    }
    const QP q = uintx_qparams(__uint_as_float(__float_as_uint(mni) & 0xFFFF0000u),
                               __uint_as_float(__float_as_uint(mxi) & 0xFFFF0000u), qmax);
    const uint32_t g = (i * L1 + (p - i * kLanePos)) / 64;
    scales[g] = (uint16_t)(__float_as_uint(q.s) >> 16);
    zeros[g] = (uint8_t)q.zp;
    qp_lds[threadIdx.x] = (__float_as_uint(q.inv) & 0xFFFF0000u) | (uint32_t)q.zp;
  }
  __syncthreads();
  if (!active) return;
  const uint32_t* qpo = &qp_lds[threadIdx.x & ~7u];
  uint32_t clo[8], chi[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t w = qpo[j];
    codes8(raw[j], __uint_as_float(w & 0xFFFF0000u), (float)(w & 0xFFu), qmax, clo[j], chi[j]);
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
template <int NB, int SINK, bool CONTIG, typename TOut>
__global__ __launch_bounds__(256) void uintx_dequant_tiled(const uint8_t* __restrict__ packed,
                                                           const uint16_t* __restrict__ scales,
                                                           const uint8_t* __restrict__ zeros, FastDiv kdiv,
                                                           uint32_t L1, Shards sh, TOut* __restrict__ out,
                                                           int64_t ldo, const uint16_t* __restrict__ W, int64_t ldw,
                                                           double* __restrict__ part) {
  using SB = ShardBits<NB>;
  __shared__ uint32_t qp_lds[256];
  const int lane = threadIdx.x & 63;
  const uint32_t p = blockIdx.x * kBlockPos + (threadIdx.x >> 6) * kWavePos + lane * kLanePos;
  const bool active = p < L1;
  uint2 s4[4], s2[2], s1;
  U4 wr[8];                                  // the error sink's weights
  if (active) {
    // The group's scale and zero point go first: the LDS exchange waits only for them,
    // while the shard bytes and the weights stay in flight across the barrier.
    const int i = lane & 7;
    const uint32_t g = (i * L1 + (p - i * kLanePos)) / 64;
    const uint32_t sc = scales[g], zz = zeros[g];
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
      for (int j = 0; j < 8; ++j) wr[j] = ld16_nt(elem_ptr<CONTIG>(W, ldw, j * L1 + p, kdiv));
    }
    qp_lds[threadIdx.x] = (sc << 16) | zz;
  }
  __syncthreads();
  double sw = 0.0, se = 0.0;
  if (active) {
    const uint32_t* qpo = &qp_lds[threadIdx.x & ~7u];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w = qpo[j];
      const float s = __uint_as_float(w & 0xFFFF0000u), zp = (float)(w & 0xFFu);
      uint32_t c[2] = {0u, 0u};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if constexpr (SB::has4) c[h] |= ((h ? s4[j & 3].y : s4[j & 3].x) >> (4 * (j >> 2))) & 0x0F0F0F0Fu;
        if constexpr (SB::has2) c[h] |= (((h ? s2[j & 1].y : s2[j & 1].x) >> (2 * (j >> 1))) & 0x03030303u) << SB::off2;
        if constexpr (SB::has1) c[h] |= (((h ? s1.y : s1.x) >> j) & 0x01010101u) << SB::off1;
      }
      float d[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) d[b] = ((float)((c[b >> 2] >> (8 * (b & 3))) & 0xFFu) - zp) * s;   // exact
      const uint32_t e = j * L1 + p;
      if constexpr (SINK == kStore && sizeof(TOut) == 2) {
        U4 v;
        v.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(ux_f32x2_t{d[0], d[1]}, ux_bf16x2_t));
        v.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(ux_f32x2_t{d[2], d[3]}, ux_bf16x2_t));
        v.z = __builtin_bit_cast(uint32_t, __builtin_convertvector(ux_f32x2_t{d[4], d[5]}, ux_bf16x2_t));
        v.w = __builtin_bit_cast(uint32_t, __builtin_convertvector(ux_f32x2_t{d[6], d[7]}, ux_bf16x2_t));
        st16_nt(elem_ptr<CONTIG>(out, ldo, e, kdiv), v);
        continue;
      }
#pragma unroll
      for (int b = 0; b < 8; b += 2) round_bf16_pair(d[b], d[b + 1]);
      if constexpr (SINK == kStore) {
        store8(elem_ptr<CONTIG>(out, ldo, e, kdiv), d);
      } else {
        float x[8];
        to_f32(Raw8<uint16_t>{wr[j]}, x);
        acc_err8(x, d, sw, se);
      }
    }
  }
  if constexpr (SINK == kErr) block_sum2_store<256>(sw, se, part);
}

// ------------------------------------------------------------- decode GEMV
// y[b, n] = sum_k x[b, k] * w[n, k] with w = bf16((q - zp) * s), the bf16 weight the
// page's forward builds before its linear. With N % 8 == 0 and K % 512 == 0, position p
// of segment j is row j * N/8 + p / K, column p % K: a lane's 8 positions of the 8
// segments share 8 activation columns and feed 8 output rows. A wavefront takes CH
// consecutive 512-position chunks of one row (CH = 4 when K % 2048 == 0), so each lane
// sums 64 * CH weights per row before one transposed reduction leaves lane j with row
// j's sum. The weight pairs (the hardware bf16 pair conversion of the exact products)
// meet the activation pairs in v_dot2c_f32_bf16; each wavefront writes one partial per
// row, added over the K / (512 CH) wavefronts of a row in order afterwards.
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

template <int NB, int B, int CH>
__global__ __launch_bounds__(256) void uintx_gemv_tiled(const uint8_t* __restrict__ packed,
                                                        const uint16_t* __restrict__ scales,
                                                        const uint8_t* __restrict__ zeros, FastDiv kdiv, uint32_t L1,
                                                        Shards sh, int N, const uint16_t* __restrict__ x,
                                                        int64_t ldx, int Bn, float* __restrict__ part) {
  using SB = ShardBits<NB>;
  __shared__ uint32_t qp_lds[CH][256];
  const int lane = threadIdx.x & 63;
  const uint32_t p0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * (uint32_t)(kWavePos * CH) + lane * kLanePos;
  const bool active = p0 < L1;               // whole wavefronts: L1 % (512 CH) == 0
  const uint32_t pa = active ? p0 : 0;
  const uint32_t row = fdiv(pa, kdiv), col0 = pa - row * kdiv.d;   // the CH chunks stay in this row
  uint2 s4[CH][4], s2[CH][2], s1[CH];
  U4 xv[CH][B];
  if (active) {
    const int i = lane & 7;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint32_t p = p0 + c * kWavePos;
      const uint32_t g = (i * L1 + (p - i * kLanePos)) / 64;
      const uint32_t sc = scales[g], zz = zeros[g];
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
      qp_lds[c][threadIdx.x] = (sc << 16) | zz;
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
    const uint32_t* qpo = &qp_lds[c][threadIdx.x & ~7u];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w = qpo[j];
      const float s = __uint_as_float(w & 0xFFFF0000u), zp = (float)(w & 0xFFu);
      uint32_t cd[2] = {0u, 0u};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if constexpr (SB::has4) cd[h] |= ((h ? s4[c][j & 3].y : s4[c][j & 3].x) >> (4 * (j >> 2))) & 0x0F0F0F0Fu;
        if constexpr (SB::has2)
          cd[h] |= (((h ? s2[c][j & 1].y : s2[c][j & 1].x) >> (2 * (j >> 1))) & 0x03030303u) << SB::off2;
        if constexpr (SB::has1) cd[h] |= (((h ? s1[c].y : s1[c].x) >> j) & 0x01010101u) << SB::off1;
      }
      const float nzs = -(zp * s);
      float d[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) d[q] = __builtin_fmaf((float)((cd[q >> 2] >> (8 * (q & 3))) & 0xFFu), s, nzs);  // exact
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
    if (lane < 8 && b < Bn) part[((int64_t)chunk * Bn + b) * N + j * (uint32_t)(N / 8) + row] = v;
  }
}

// ------------------------------------------------------------------ launchers
bool uintx_tiled(int32_t dt, int group, int64_t N, int64_t K) {
  return dt == kBF16 && group == 64 && ((N * K) % 512) == 0;
}
size_t uintx_code_workspace(int32_t dt, int group, int64_t N, int64_t K) {
  return uintx_tiled(dt, group, N, K) ? 0 : (size_t)(N * K);
}

static unsigned tiles_of(int64_t N, int64_t K) { return (unsigned)(((uint64_t)(N * K) / 8 + kBlockPos - 1) / kBlockPos); }

template <int NB>
static void quant_tiled(const void* W, int64_t N, int64_t K, int64_t ldw, void* packed, void* scales, void* zeros,
                        hipStream_t st) {
  const uint32_t numel = (uint32_t)(N * K);
  const Shards sh = shards_of(NB, numel);
  const FastDiv kdiv = make_fastdiv((uint32_t)K);
  hipLaunchKernelGGL((ldw == K ? uintx_quant_tiled<NB, true> : uintx_quant_tiled<NB, false>), dim3(tiles_of(N, K)),
                     dim3(256), 0, st, (const uint16_t*)W, ldw, kdiv, numel / 8, sh, (uint8_t*)packed,
                     (uint16_t*)scales, (uint8_t*)zeros);
}

void launch_uintx_quant(int nbits, int32_t dt, int group, const void* W, int64_t N, int64_t K, int64_t ldw,
                        void* packed, void* scales, void* zeros, void* workspace, hipStream_t st) {
  if (!uintx_tiled(dt, group, N, K)) {
    launch_uintx_quant_flat(nbits, dt, group, W, N, K, ldw, packed, scales, zeros, workspace, st);
    return;
  }
  switch (nbits) {
    case 2: quant_tiled<2>(W, N, K, ldw, packed, scales, zeros, st); break;
    case 3: quant_tiled<3>(W, N, K, ldw, packed, scales, zeros, st); break;
    case 4: quant_tiled<4>(W, N, K, ldw, packed, scales, zeros, st); break;
    case 5: quant_tiled<5>(W, N, K, ldw, packed, scales, zeros, st); break;
    case 6: quant_tiled<6>(W, N, K, ldw, packed, scales, zeros, st); break;
    default: quant_tiled<7>(W, N, K, ldw, packed, scales, zeros, st); break;
  }
}

template <int NB, int SINK, typename TOut>
static void deq_tiled(const void* packed, const void* scales, const void* zeros, int64_t N, int64_t K, void* out,
                      int64_t ldo, const void* W, int64_t ldw, double* part, hipStream_t st) {
  const uint32_t numel = (uint32_t)(N * K);
  const Shards sh = shards_of(NB, numel);
  const FastDiv kdiv = make_fastdiv((uint32_t)K);
  const bool contig = SINK == kStore ? ldo == K : ldw == K;
  hipLaunchKernelGGL((contig ? uintx_dequant_tiled<NB, SINK, true, TOut> : uintx_dequant_tiled<NB, SINK, false, TOut>),
                     dim3(tiles_of(N, K)), dim3(256), 0, st, (const uint8_t*)packed, (const uint16_t*)scales,
                     (const uint8_t*)zeros, kdiv, numel / 8, sh, (TOut*)out, ldo, (const uint16_t*)W, ldw, part);
}

template <int SINK, typename TOut>
static void deq_tiled_nb(int nbits, const void* packed, const void* scales, const void* zeros, int64_t N, int64_t K,
                         void* out, int64_t ldo, const void* W, int64_t ldw, double* part, hipStream_t st) {
  switch (nbits) {
    case 2: deq_tiled<2, SINK, TOut>(packed, scales, zeros, N, K, out, ldo, W, ldw, part, st); break;
    case 3: deq_tiled<3, SINK, TOut>(packed, scales, zeros, N, K, out, ldo, W, ldw, part, st); break;
    case 4: deq_tiled<4, SINK, TOut>(packed, scales, zeros, N, K, out, ldo, W, ldw, part, st); break;
    case 5: deq_tiled<5, SINK, TOut>(packed, scales, zeros, N, K, out, ldo, W, ldw, part, st); break;
    case 6: deq_tiled<6, SINK, TOut>(packed, scales, zeros, N, K, out, ldo, W, ldw, part, st); break;
    default: deq_tiled<7, SINK, TOut>(packed, scales, zeros, N, K, out, ldo, W, ldw, part, st); break;
  }
}

void launch_uintx_dequant(int nbits, int32_t dt, int group, const void* packed, const void* scales,
                          const void* zeros, int64_t N, int64_t K, void* out, int32_t out_dtype, int64_t ldo,
                          hipStream_t st) {
  if (!uintx_tiled(dt, group, N, K))
    launch_uintx_dequant_flat(nbits, dt, group, packed, scales, zeros, N, K, out, out_dtype, ldo, st);
  else if (out_dtype == kBF16)
    deq_tiled_nb<kStore, uint16_t>(nbits, packed, scales, zeros, N, K, out, ldo, nullptr, 0, nullptr, st);
  else
    deq_tiled_nb<kStore, float>(nbits, packed, scales, zeros, N, K, out, ldo, nullptr, 0, nullptr, st);
}

// The tiled error kernel runs one block per tile (its partials follow the tiles); the
// flat one is grid-stride with a capped grid. Both depend on the shape only.
unsigned uintx_err_blocks(int32_t dt, int group, int64_t N, int64_t K) {
  return uintx_tiled(dt, group, N, K) ? tiles_of(N, K) : uintx_flat_err_blocks(N, K);
}

void launch_uintx_err(int nbits, int32_t dt, int group, const void* W, int64_t N, int64_t K, int64_t ldw,
                      const void* packed, const void* scales, const void* zeros, double* part, hipStream_t st) {
  if (uintx_tiled(dt, group, N, K))
    deq_tiled_nb<kErr, float>(nbits, packed, scales, zeros, N, K, nullptr, 0, W, ldw, part, st);
  else
    launch_uintx_err_flat(nbits, dt, group, W, N, K, ldw, packed, scales, zeros, part, st);
}

}  // namespace gwb

namespace gwb {

template <int NB, int B, int CH>
static void gemv_tiled(int Bn, const void* packed, const void* scales, const void* zeros, int64_t N, int64_t K,
                       const void* x, int64_t ldx, float* part, hipStream_t st) {
  const uint32_t numel = (uint32_t)(N * K);
  const unsigned blocks = (unsigned)(((uint64_t)numel / 8 / (kWavePos * CH) + 3) / 4);
  hipLaunchKernelGGL((uintx_gemv_tiled<NB, B, CH>), dim3(blocks), dim3(256), 0, st, (const uint8_t*)packed,
                     (const uint16_t*)scales, (const uint8_t*)zeros, make_fastdiv((uint32_t)K), numel / 8,
                     shards_of(NB, numel), (int)N, (const uint16_t*)x, ldx, Bn, part);
}

template <int NB, int CH>
static void gemv_ch(int B, const void* packed, const void* scales, const void* zeros, int64_t N, int64_t K,
                    const void* x, int64_t ldx, float* part, hipStream_t st) {
  if (B == 1) gemv_tiled<NB, 1, CH>(B, packed, scales, zeros, N, K, x, ldx, part, st);
  else if (B == 2) gemv_tiled<NB, 2, CH>(B, packed, scales, zeros, N, K, x, ldx, part, st);
  else if (B <= 4) gemv_tiled<NB, 4, CH>(B, packed, scales, zeros, N, K, x, ldx, part, st);
  else gemv_tiled<NB, 8, CH>(B, packed, scales, zeros, N, K, x, ldx, part, st);
}

template <int NB>
static void gemv_nb(int B, const void* packed, const void* scales, const void* zeros, int64_t N, int64_t K,
                    const void* x, int64_t ldx, float* part, hipStream_t st) {
  if (K % 2048 == 0) gemv_ch<NB, 4>(B, packed, scales, zeros, N, K, x, ldx, part, st);
  else gemv_ch<NB, 1>(B, packed, scales, zeros, N, K, x, ldx, part, st);
}

int uintx_gemv_splits(int64_t K) { return (int)(K % 2048 == 0 ? K / 2048 : K / 512); }

bool uintx_gemv_supported(int64_t N, int64_t K) { return N % 8 == 0 && K % 512 == 0; }

void launch_uintx_gemv(int nbits, int B, const void* packed, const void* scales, const void* zeros, int64_t N,
                       int64_t K, const void* x, int64_t ldx, void* y, int32_t y_dtype, int64_t ldy, float* part,
                       hipStream_t st) {
  switch (nbits) {
    case 2: gemv_nb<2>(B, packed, scales, zeros, N, K, x, ldx, part, st); break;
    case 3: gemv_nb<3>(B, packed, scales, zeros, N, K, x, ldx, part, st); break;
    case 4: gemv_nb<4>(B, packed, scales, zeros, N, K, x, ldx, part, st); break;
    case 5: gemv_nb<5>(B, packed, scales, zeros, N, K, x, ldx, part, st); break;
    case 6: gemv_nb<6>(B, packed, scales, zeros, N, K, x, ldx, part, st); break;
    default: gemv_nb<7>(B, packed, scales, zeros, N, K, x, ldx, part, st); break;
  }
  launch_gemv_finalize(part, uintx_gemv_splits(K), B, N, y, y_dtype, ldy, st);
}

}  // namespace gwb
