// Affine uint2..uint7 (torchao-style, preserve_zero, bfloat16 arithmetic) quantize+
// pack into planar power-of-two shards, unpack+dequantize, fused reconstruction error.
// Page uintx_quant.py: _pack_shard, pack_uintx, unpack_uintx,
// UIntXQuantizer._quantize_impl and _dequantize_native. Group 64 along K.
//
// Planar shards: byte i of the k-bit shard holds codes i, i+L, i+2L, ... (L = that
// shard's byte count), which lie far apart in the matrix. With numel % 512 == 0 the
// shard lengths nest (L_1 = numel/8, L_2 = 2 L_1, L_4 = 4 L_1), so a block that takes
// the 8 segments [b0 + j*L_1, b0 + j*L_1 + T), j = 0..7, owns complete bytes of every
// shard: [b0, b0+T) of the 1-bit shard, [b0 + m*L_1, +T) for m < 2 of the 2-bit
// shard and for m < 4 of the 4-bit shard. Segments start on group boundaries, so
// qparams stay local. Codes meet in LDS, where bytes are assembled four at a time.
// Other sizes take a two-pass path: codes to workspace, then one thread per byte.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gwb {

constexpr int kT = 256;          // elements per segment per block
constexpr int kCS = kT + 16;     // LDS row stride of the code tile (bytes)

struct Shards {                  // byte offsets and bit offsets of the present shards
  int64_t base4, base2, base1;
  int off2, off1;
  bool has4, has2, has1;
};
static Shards shards_of(int nbits, int64_t numel) {
  Shards s{};
  s.has4 = nbits & 4; s.has2 = nbits & 2; s.has1 = nbits & 1;
  int64_t L4 = (numel + 1) / 2, L2 = (numel + 3) / 4;
  s.base4 = 0;
  s.base2 = s.has4 ? L4 : 0;
  s.base1 = s.base2 + (s.has2 ? L2 : 0);
  s.off2 = s.has4 ? 4 : 0;
  s.off1 = (s.has4 ? 4 : 0) + (s.has2 ? 2 : 0);
  return s;
}

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

// Load 8 consecutive bf16 of flat element e (row-major [N, K], row stride ldw).
__device__ __forceinline__ void load8_at(const uint16_t* W, int64_t ldw, uint32_t e, FastDiv kdiv, float* x) {
  uint32_t n = fdiv(e, kdiv);
  uint32_t k = e - n * kdiv.d;
  load8(W + (int64_t)n * ldw + k, x);
}

// ------------------------------------------------------------- tiled quantize
__global__ __launch_bounds__(256) void uintx_quant_tiled(const uint16_t* __restrict__ W, int64_t ldw,
                                                         FastDiv kdiv, uint32_t L1, int nbits, Shards sh,
                                                         uint8_t* __restrict__ packed,
                                                         uint16_t* __restrict__ scales,
                                                         uint8_t* __restrict__ zeros) {
  __shared__ uint8_t ctile[8 * kCS];
  const int t = threadIdx.x;
  const uint32_t b0 = blockIdx.x * kT;
  const uint32_t Tb = min((uint32_t)kT, L1 - b0);      // a multiple of 64
  const float qmax = (float)((1 << nbits) - 1);
  {
    const int j = t / 32, tl = t % 32;
    if ((uint32_t)tl * 8 < Tb) {
      const uint32_t e = j * L1 + b0 + tl * 8;
      float x[8];
      load8_at(W, ldw, e, kdiv, x);
      float mn = x[0], mx = x[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) { mn = fminf(mn, x[i]); mx = fmaxf(mx, x[i]); }
      mn = lanes_min<8>(mn);
      mx = lanes_max<8>(mx);
      QP q = uintx_qparams(mn, mx, qmax);
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) lo |= uintx_code(x[i], q, qmax) << (8 * i);
#pragma unroll
      for (int i = 0; i < 4; ++i) hi |= uintx_code(x[i + 4], q, qmax) << (8 * i);
      uint32_t* dst = reinterpret_cast<uint32_t*>(&ctile[j * kCS + tl * 8]);
      dst[0] = lo;
      dst[1] = hi;
      if ((tl & 7) == 0) {
        const uint32_t gi = e / 64;
        scales[gi] = (uint16_t)(__float_as_uint(q.s) >> 16);
        zeros[gi] = (uint8_t)q.zp;
      }
    }
  }
  __syncthreads();
  const int rho = t / 64;
  const uint32_t p4 = (t % 64) * 4;
  if (p4 >= Tb) return;
  uint32_t C[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) C[j] = *reinterpret_cast<const uint32_t*>(&ctile[j * kCS + p4]);
  if (sh.has4) {
    const int m = rho;
    uint32_t v = (C[m] & 0x0F0F0F0Fu) | ((C[m + 4] & 0x0F0F0F0Fu) << 4);
    *reinterpret_cast<uint32_t*>(packed + sh.base4 + (int64_t)m * L1 + b0 + p4) = v;
  }
  if (sh.has2 && rho < 2) {
    const int m = rho;
    uint32_t v = 0;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) v |= ((C[m + 2 * jj] >> sh.off2) & 0x03030303u) << (2 * jj);
    *reinterpret_cast<uint32_t*>(packed + sh.base2 + (int64_t)m * L1 + b0 + p4) = v;
  }
  if (sh.has1 && rho == 0) {
    uint32_t v = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) v |= ((C[j] >> sh.off1) & 0x01010101u) << j;
    *reinterpret_cast<uint32_t*>(packed + sh.base1 + b0 + p4) = v;
  }
}

// ------------------------------------------------------------- tiled dequantize
template <int SINK, typename TOut>
__global__ __launch_bounds__(256) void uintx_dequant_tiled(const uint8_t* __restrict__ packed,
                                                           const uint16_t* __restrict__ scales,
                                                           const uint8_t* __restrict__ zeros,
                                                           FastDiv kdiv, uint32_t L1, int nbits, Shards sh,
                                                           TOut* __restrict__ out, int64_t ldo,
                                                           const uint16_t* __restrict__ W, int64_t ldw,
                                                           double* __restrict__ part) {
  __shared__ uint8_t s4[4 * kCS], s2[2 * kCS], s1[kCS];
  const int t = threadIdx.x;
  const int rho = t / 64;
  const uint32_t p4 = (t % 64) * 4;
  const int j = t / 32, tl = t % 32;
  double sw = 0.0, se = 0.0;
  const uint32_t ntiles = (L1 + kT - 1) / kT;
  for (uint32_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const uint32_t b0 = tile * kT;
    const uint32_t Tb = min((uint32_t)kT, L1 - b0);
    if (p4 < Tb) {
      if (sh.has4)
        *reinterpret_cast<uint32_t*>(&s4[rho * kCS + p4]) =
            *reinterpret_cast<const uint32_t*>(packed + sh.base4 + (int64_t)rho * L1 + b0 + p4);
      if (sh.has2 && rho < 2)
        *reinterpret_cast<uint32_t*>(&s2[rho * kCS + p4]) =
            *reinterpret_cast<const uint32_t*>(packed + sh.base2 + (int64_t)rho * L1 + b0 + p4);
      if (sh.has1 && rho == 0)
        *reinterpret_cast<uint32_t*>(&s1[p4]) = *reinterpret_cast<const uint32_t*>(packed + sh.base1 + b0 + p4);
    }
    __syncthreads();
    if ((uint32_t)tl * 8 < Tb) {
      const uint32_t e = j * L1 + b0 + tl * 8;
      const uint32_t gi = e / 64;
      const float s = bf16_to_f32(scales[gi]);
      const float zp = (float)zeros[gi];
      float d[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int p = tl * 8 + i;
        uint32_t c = 0;
        if (sh.has4) c |= (s4[(j & 3) * kCS + p] >> (4 * (j >> 2))) & 0xFu;
        if (sh.has2) c |= ((s2[(j & 1) * kCS + p] >> (2 * (j >> 1))) & 0x3u) << sh.off2;
        if (sh.has1) c |= ((s1[p] >> j) & 0x1u) << sh.off1;
        d[i] = uintx_value(c, zp, s);
      }
      const uint32_t n = fdiv(e, kdiv);
      const uint32_t k = e - n * kdiv.d;
      if constexpr (SINK == kStore) {
        store8(out + (int64_t)n * ldo + k, d);
      } else {
        float x[8];
        load8(W + (int64_t)n * ldw + k, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          double xd = (double)x[i];
          double ed = (double)(x[i] - d[i]);
          sw = fma(xd, xd, sw);
          se = fma(ed, ed, se);
        }
      }
    }
    __syncthreads();
  }
  if constexpr (SINK == kErr) block_sum2_store<256>(sw, se, part);
}

// ------------------------------------------------------------- ragged sizes
// Pass 1: codes of 8 consecutive elements per lane (8 lanes per group) to workspace.
__global__ __launch_bounds__(256) void uintx_codes_flat(const uint16_t* __restrict__ W, int64_t ldw,
                                                        FastDiv kdiv, uint32_t units, int nbits,
                                                        uint8_t* __restrict__ codes,
                                                        uint16_t* __restrict__ scales,
                                                        uint8_t* __restrict__ zeros) {
  const float qmax = (float)((1 << nbits) - 1);
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
    float x[8];
    load8_at(W, ldw, u * 8, kdiv, x);
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) { mn = fminf(mn, x[i]); mx = fmaxf(mx, x[i]); }
    mn = lanes_min<8>(mn);
    mx = lanes_max<8>(mx);
    QP q = uintx_qparams(mn, mx, qmax);
#pragma unroll
    for (int i = 0; i < 8; ++i) codes[u * 8 + i] = (uint8_t)uintx_code(x[i], q, qmax);
    if ((u & 7u) == 0) {
      scales[u / 8] = (uint16_t)(__float_as_uint(q.s) >> 16);
      zeros[u / 8] = (uint8_t)q.zp;
    }
  }
}

// Pass 2: one thread per byte of the k-bit shard (bits [off, off+k) of each code).
__global__ __launch_bounds__(256) void uintx_pack_shard(const uint8_t* __restrict__ codes, uint32_t numel,
                                                        int k, int off, uint8_t* __restrict__ shard) {
  const int vpb = 8 / k;
  const uint32_t L = (numel + vpb - 1) / vpb;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < L; i += stride) {
    uint32_t v = 0;
    for (int j = 0; j < vpb; ++j) {
      uint32_t idx = j * L + i;
      if (idx < numel) v |= ((codes[idx] >> off) & ((1u << k) - 1u)) << (j * k);
    }
    shard[i] = (uint8_t)v;
  }
}

__device__ __forceinline__ uint32_t uintx_gather(const uint8_t* packed, const Shards& sh, uint32_t numel,
                                                 uint32_t idx) {
  uint32_t c = 0;
  if (sh.has4) {
    uint32_t L = (numel + 1) / 2;
    c |= (packed[sh.base4 + idx % L] >> (4 * (idx / L))) & 0xFu;
  }
  if (sh.has2) {
    uint32_t L = (numel + 3) / 4;
    c |= ((packed[sh.base2 + idx % L] >> (2 * (idx / L))) & 0x3u) << sh.off2;
  }
  if (sh.has1) {
    uint32_t L = (numel + 7) / 8;
    c |= ((packed[sh.base1 + idx % L] >> (idx / L)) & 0x1u) << sh.off1;
  }
  return c;
}

template <int SINK, typename TOut>
__global__ __launch_bounds__(256) void uintx_dequant_flat(const uint8_t* __restrict__ packed,
                                                          const uint16_t* __restrict__ scales,
                                                          const uint8_t* __restrict__ zeros,
                                                          FastDiv kdiv, uint32_t units, uint32_t numel,
                                                          Shards sh, TOut* __restrict__ out, int64_t ldo,
                                                          const uint16_t* __restrict__ W, int64_t ldw,
                                                          double* __restrict__ part) {
  const uint32_t stride = gridDim.x * blockDim.x;
  double sw = 0.0, se = 0.0;
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
    const uint32_t e = u * 8;
    const float s = bf16_to_f32(scales[e / 64]);
    const float zp = (float)zeros[e / 64];
    float d[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = uintx_value(uintx_gather(packed, sh, numel, e + i), zp, s);
    const uint32_t n = fdiv(e, kdiv);
    const uint32_t k = e - n * kdiv.d;
    if constexpr (SINK == kStore) {
      store8(out + (int64_t)n * ldo + k, d);
    } else {
      float x[8];
      load8(W + (int64_t)n * ldw + k, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        double xd = (double)x[i];
        double ed = (double)(x[i] - d[i]);
        sw = fma(xd, xd, sw);
        se = fma(ed, ed, se);
      }
    }
  }
  if constexpr (SINK == kErr) block_sum2_store<256>(sw, se, part);
}

// ------------------------------------------------------------------ launchers
bool uintx_tiled(int64_t N, int64_t K) { return ((N * K) % 512) == 0; }
size_t uintx_code_workspace(int64_t N, int64_t K) { return uintx_tiled(N, K) ? 0 : (size_t)(N * K); }

static unsigned capped(uint64_t blocks, unsigned cap) {
  return (unsigned)(blocks < cap ? (blocks ? blocks : 1) : cap);
}

void launch_uintx_quant(int nbits, const void* W, int64_t N, int64_t K, int64_t ldw, void* packed,
                        void* scales, void* zeros, void* workspace, hipStream_t st) {
  const uint32_t numel = (uint32_t)(N * K);
  const Shards sh = shards_of(nbits, numel);
  const FastDiv kdiv = make_fastdiv((uint32_t)K);
  if (uintx_tiled(N, K)) {
    const uint32_t L1 = numel / 8;
    hipLaunchKernelGGL(uintx_quant_tiled, dim3((L1 + kT - 1) / kT), dim3(256), 0, st, (const uint16_t*)W, ldw,
                       kdiv, L1, nbits, sh, (uint8_t*)packed, (uint16_t*)scales, (uint8_t*)zeros);
    return;
  }
  uint8_t* codes = (uint8_t*)workspace;
  const uint32_t units = numel / 8;
  hipLaunchKernelGGL(uintx_codes_flat, dim3(capped((units + 255) / 256, kStreamGridCap)), dim3(256), 0, st,
                     (const uint16_t*)W, ldw, kdiv, units, nbits, codes, (uint16_t*)scales, (uint8_t*)zeros);
  int off = 0;
  for (int k : {4, 2, 1}) {
    if (!(nbits & k)) continue;
    int64_t base = k == 4 ? sh.base4 : (k == 2 ? sh.base2 : sh.base1);
    uint32_t L = (numel + (8 / k) - 1) / (8 / k);
    hipLaunchKernelGGL(uintx_pack_shard, dim3(capped((L + 255) / 256, kStreamGridCap)), dim3(256), 0, st,
                       (const uint8_t*)codes, numel, k, off, (uint8_t*)packed + base);
    off += k;
  }
}

template <int SINK, typename TOut>
static void deq(unsigned grid, int nbits, const void* packed, const void* scales, const void* zeros, int64_t N,
                int64_t K, void* out, int64_t ldo, const void* W, int64_t ldw, double* part, hipStream_t st) {
  const uint32_t numel = (uint32_t)(N * K);
  const Shards sh = shards_of(nbits, numel);
  const FastDiv kdiv = make_fastdiv((uint32_t)K);
  if (uintx_tiled(N, K)) {
    hipLaunchKernelGGL((uintx_dequant_tiled<SINK, TOut>), dim3(grid), dim3(256), 0, st, (const uint8_t*)packed,
                       (const uint16_t*)scales, (const uint8_t*)zeros, kdiv, numel / 8, nbits, sh, (TOut*)out,
                       ldo, (const uint16_t*)W, ldw, part);
  } else {
    hipLaunchKernelGGL((uintx_dequant_flat<SINK, TOut>), dim3(grid), dim3(256), 0, st, (const uint8_t*)packed,
                       (const uint16_t*)scales, (const uint8_t*)zeros, kdiv, numel / 8, numel, sh, (TOut*)out,
                       ldo, (const uint16_t*)W, ldw, part);
  }
}

static uint64_t uintx_blocks(int64_t N, int64_t K) {
  uint64_t numel = (uint64_t)(N * K);
  return uintx_tiled(N, K) ? (numel / 8 + kT - 1) / kT : (numel / 8 + 255) / 256;
}

void launch_uintx_dequant(int nbits, const void* packed, const void* scales, const void* zeros,
                          int64_t N, int64_t K, void* out, int32_t out_dtype, int64_t ldo,
                          hipStream_t st) {
  unsigned grid = capped(uintx_blocks(N, K), kStreamGridCap);
  if (out_dtype == kBF16)
    deq<kStore, uint16_t>(grid, nbits, packed, scales, zeros, N, K, out, ldo, nullptr, 0, nullptr, st);
  else
    deq<kStore, float>(grid, nbits, packed, scales, zeros, N, K, out, ldo, nullptr, 0, nullptr, st);
}

unsigned uintx_err_blocks(int64_t N, int64_t K) { return capped(uintx_blocks(N, K), kErrGridCap); }

void launch_uintx_err(int nbits, const void* W, int64_t N, int64_t K, int64_t ldw, const void* packed,
                      const void* scales, const void* zeros, double* part, hipStream_t st) {
  deq<kErr, float>(uintx_err_blocks(N, K), nbits, packed, scales, zeros, N, K, nullptr, 0, W, ldw, part, st);
}

}  // namespace gwb
