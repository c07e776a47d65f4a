// Affine uint2..uint7 (torchao-style, preserve_zero): the bfloat16 / group-64 tiled
// kernels (page uintx_quant.py's defaults), the decode GEMV on packed uintx weights, and
// the launch selection for every dtype and group. Page uintx_quant.py: pack_uintx,
// unpack_uintx, UIntXQuantizer._quantize_impl, _dequantize_native and forward.
// The tiled kernels (uintx_tiled.hpp) need numel % 8G == 0; their other instantiations
// live in uintx_f16.hip, uintx_f32.hip and uintx_bf16.hip, and every other shape takes
// the two-pass path of uintx_flat.hip.
#include "device_common.hpp"
#include "kernels.hpp"
#include "uintx_layout.hpp"
#include "uintx_tiled.hpp"

namespace gwb {

// ------------------------------------------------------------- decode GEMV
// y[b, n] = sum_k x[b, k] * w[n, k] with w = bf16((q - zp) * s), the bf16 weight the
// page's forward builds before its linear. With N % 8 == 0 and K % 512 == 0, position p
// of segment j is row j * N/8 + p / K, column p % K: a lane's 8 positions of the 8
// segments share 8 activation columns and feed 8 output rows. A wavefront takes CH
// consecutive 512-position chunks of one row (CH = 4 when K % 2048 == 0), so each lane
// sums 64 * CH weights per row before one transposed reduction leaves lane j with row
// j's sum. The weight pairs (the hardware bf16 pair conversion of the exact products)
// meet the activation pairs in v_dot2c_f32_bf16; each wavefront writes one partial per
// row, added over the K / (512 CH) wavefronts of a row in order afterwards, or, when one
// wavefront covers the whole row, the row's sum straight into y.
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

// Where the GEMV's row sums go: K-split partials, or y itself (float32 or bf16, RNE).
struct GemvOut {
  enum { kPart = 0, kF32 = 1, kBF16 = 2 };
  float* part;
  void* y;
  int64_t ldy;
  int mode;
};

template <int NB, int B, int CH>
__global__ __launch_bounds__(256) void uintx_gemv_tiled(const uint8_t* __restrict__ packed,
                                                        const uint16_t* __restrict__ scales,
                                                        const uint8_t* __restrict__ zeros, FastDiv kdiv, uint32_t L1,
                                                        Shards sh, int N, const uint16_t* __restrict__ x,
                                                        int64_t ldx, int Bn, GemvOut out) {
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
    if (lane < 8 && b < Bn) {
      const int64_t n = (int64_t)j * (N / 8) + row;
      if (out.mode == GemvOut::kPart) out.part[((int64_t)chunk * Bn + b) * N + n] = v;
      else if (out.mode == GemvOut::kF32) static_cast<float*>(out.y)[b * out.ldy + n] = v;
      else static_cast<uint16_t*>(out.y)[b * out.ldy + n] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

// ------------------------------------------------------------------ launchers
bool uintx_tiled(int32_t dt, int group, int64_t N, int64_t K) {
  (void)dt;
  return uintx_tiles_fit(group, N * K);
}
size_t uintx_code_workspace(int32_t dt, int group, int64_t N, int64_t K) {
  return uintx_tiled(dt, group, N, K) ? 0 : (size_t)(N * K);
}

void launch_uintx_quant(int nbits, int32_t dt, int group, const void* W, int64_t N, int64_t K, int64_t ldw,
                        void* packed, void* scales, void* zeros, void* workspace, hipStream_t st) {
  if (!uintx_tiled(dt, group, N, K))
    launch_uintx_quant_flat(nbits, dt, group, W, N, K, ldw, packed, scales, zeros, workspace, st);
  else if (dt == kBF16 && group == 64)
    ux_tiled_quant_entry<kBF16, 64>(nbits, W, N, K, ldw, packed, scales, zeros, st);
  else if (dt == kBF16)
    uintx_tiled_quant_bf16(nbits, group, W, N, K, ldw, packed, scales, zeros, st);
  else if (dt == kF16)
    uintx_tiled_quant_f16(nbits, group, W, N, K, ldw, packed, scales, zeros, st);
  else
    uintx_tiled_quant_f32(nbits, group, W, N, K, ldw, packed, scales, zeros, st);
}

void launch_uintx_dequant(int nbits, int32_t dt, int group, const void* packed, const void* scales,
                          const void* zeros, int64_t N, int64_t K, void* out, int32_t out_dtype, int64_t ldo,
                          hipStream_t st) {
  if (!uintx_tiled(dt, group, N, K))
    launch_uintx_dequant_flat(nbits, dt, group, packed, scales, zeros, N, K, out, out_dtype, ldo, st);
  else if (dt == kBF16 && group == 64)
    ux_tiled_dequant_entry<kBF16, 64>(nbits, packed, scales, zeros, N, K, out, out_dtype, ldo, st);
  else if (dt == kBF16)
    uintx_tiled_dequant_bf16(nbits, group, packed, scales, zeros, N, K, out, out_dtype, ldo, st);
  else if (dt == kF16)
    uintx_tiled_dequant_f16(nbits, group, packed, scales, zeros, N, K, out, out_dtype, ldo, st);
  else
    uintx_tiled_dequant_f32(nbits, group, packed, scales, zeros, N, K, out, out_dtype, ldo, st);
}

// The tiled error kernels run one block per tile (their partials follow the tiles); the
// flat one is grid-stride with a capped grid. Both depend on the shape only.
unsigned uintx_err_blocks(int32_t dt, int group, int64_t N, int64_t K) {
  return uintx_tiled(dt, group, N, K) ? uintx_tiles(N * K) : uintx_flat_err_blocks(N, K);
}

void launch_uintx_err(int nbits, int32_t dt, int group, const void* W, int64_t N, int64_t K, int64_t ldw,
                      const void* packed, const void* scales, const void* zeros, double* part, hipStream_t st) {
  if (!uintx_tiled(dt, group, N, K))
    launch_uintx_err_flat(nbits, dt, group, W, N, K, ldw, packed, scales, zeros, part, st);
  else if (dt == kBF16 && group == 64)
    ux_tiled_err_entry<kBF16, 64>(nbits, W, N, K, ldw, packed, scales, zeros, part, st);
  else if (dt == kBF16)
    uintx_tiled_err_bf16(nbits, group, W, N, K, ldw, packed, scales, zeros, part, st);
  else if (dt == kF16)
    uintx_tiled_err_f16(nbits, group, W, N, K, ldw, packed, scales, zeros, part, st);
  else
    uintx_tiled_err_f32(nbits, group, W, N, K, ldw, packed, scales, zeros, part, st);
}

}  // namespace gwb

namespace gwb {

template <int NB, int B, int CH>
static void gemv_tiled(int Bn, const void* packed, const void* scales, const void* zeros, int64_t N, int64_t K,
                       const void* x, int64_t ldx, GemvOut out, hipStream_t st) {
  const uint32_t numel = (uint32_t)(N * K);
  const unsigned blocks = (unsigned)(((uint64_t)numel / 8 / (kWavePos * CH) + 3) / 4);
  hipLaunchKernelGGL((uintx_gemv_tiled<NB, B, CH>), dim3(blocks), dim3(256), 0, st, (const uint8_t*)packed,
                     (const uint16_t*)scales, (const uint8_t*)zeros, make_fastdiv((uint32_t)K), numel / 8,
                     shards_of(NB, numel), (int)N, (const uint16_t*)x, ldx, Bn, out);
}

template <int NB, int CH>
static void gemv_ch(int B, const void* packed, const void* scales, const void* zeros, int64_t N, int64_t K,
                    const void* x, int64_t ldx, GemvOut out, hipStream_t st) {
  if (B == 1) gemv_tiled<NB, 1, CH>(B, packed, scales, zeros, N, K, x, ldx, out, st);
  else if (B == 2) gemv_tiled<NB, 2, CH>(B, packed, scales, zeros, N, K, x, ldx, out, st);
  else if (B <= 4) gemv_tiled<NB, 4, CH>(B, packed, scales, zeros, N, K, x, ldx, out, st);
  else gemv_tiled<NB, 8, CH>(B, packed, scales, zeros, N, K, x, ldx, out, st);
}

template <int NB>
static void gemv_nb(int B, const void* packed, const void* scales, const void* zeros, int64_t N, int64_t K,
                    const void* x, int64_t ldx, GemvOut out, hipStream_t st) {
  if (K % 2048 == 0) gemv_ch<NB, 4>(B, packed, scales, zeros, N, K, x, ldx, out, st);
  else gemv_ch<NB, 1>(B, packed, scales, zeros, N, K, x, ldx, out, st);
}

int uintx_gemv_splits(int64_t K) { return (int)(K % 2048 == 0 ? K / 2048 : K / 512); }

bool uintx_gemv_supported(int64_t N, int64_t K) { return N % 8 == 0 && K % 512 == 0; }

void launch_uintx_gemv(int nbits, int B, const void* packed, const void* scales, const void* zeros, int64_t N,
                       int64_t K, const void* x, int64_t ldx, void* y, int32_t y_dtype, int64_t ldy, float* part,
                       hipStream_t st) {
  // one split: each row's sum is complete in one wavefront and goes straight to y
  const int S = uintx_gemv_splits(K);
  GemvOut out{part, y, ldy, S > 1 ? GemvOut::kPart : (y_dtype == kBF16 ? GemvOut::kBF16 : GemvOut::kF32)};
  switch (nbits) {
    case 2: gemv_nb<2>(B, packed, scales, zeros, N, K, x, ldx, out, st); break;
    case 3: gemv_nb<3>(B, packed, scales, zeros, N, K, x, ldx, out, st); break;
    case 4: gemv_nb<4>(B, packed, scales, zeros, N, K, x, ldx, out, st); break;
    case 5: gemv_nb<5>(B, packed, scales, zeros, N, K, x, ldx, out, st); break;
    case 6: gemv_nb<6>(B, packed, scales, zeros, N, K, x, ldx, out, st); break;
    default: gemv_nb<7>(B, packed, scales, zeros, N, K, x, ldx, out, st); break;
  }
  if (S > 1) launch_gemv_finalize(part, S, B, N, y, y_dtype, ldy, st);
}

}  // namespace gwb
