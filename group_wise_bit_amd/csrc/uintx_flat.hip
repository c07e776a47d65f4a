// Affine uint2..uint7 on any weight dtype (bfloat16, float16, float32) and group size
// (32, 64, 128): the general path beside the tiled bfloat16 / group-64 kernels of
// uintx.hip, for every shape. Page uintx_quant.py, UIntXQuantizer._quantize_impl and
// _dequantize_native: the arithmetic runs in the weight's own dtype (each op one
// float32 op rounded to that dtype; float32 weights: plain float32 ops, with the IEEE
// division the page writes for scale / qmax), and the scale is stored as that dtype.
//
// Quantization takes two passes: codes of 8 consecutive weights per lane (G/8 lanes
// per group, DPP min/max) to a workspace, then one thread per byte of each shard.
// Dequantization and the fused error sink gather each code from its shards.
// The per-dtype arithmetic (uintx_math.hpp) is shared with the tiled kernels.
#include "device_common.hpp"
#include "kernels.hpp"
#include "uintx_layout.hpp"
#include "uintx_math.hpp"

namespace gwb {

// 8 consecutive weights (16-byte aligned) as float32.
template <int DT>
__device__ __forceinline__ void load8_dt(const typename UxDt<DT>::T* p, float* x) {
  if constexpr (DT == kF32) {
    load8(p, x);
  } else {
    const U4 v = ld16(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[2 * q] = UxDt<DT>::value(w[q] & 0xFFFFu);
      x[2 * q + 1] = UxDt<DT>::value(w[q] >> 16);
    }
  }
}
template <int DT>
__device__ __forceinline__ void load8_at(const typename UxDt<DT>::T* W, int64_t ldw, uint32_t e, FastDiv kdiv,
                                         float* x) {
  const uint32_t n = fdiv(e, kdiv);
  load8_dt<DT>(W + (int64_t)n * ldw + (e - n * kdiv.d), x);
}

// Pass 1: codes of 8 consecutive elements per lane to workspace, G/8 lanes per group.
// Grid-stride: the stride and units are multiples of G/8, so a group's lanes stay
// together in every iteration.
template <int DT, int G>
__global__ __launch_bounds__(256) void uintx_codes_flat(const typename UxDt<DT>::T* __restrict__ W, int64_t ldw,
                                                        FastDiv kdiv, uint32_t units, int nbits,
                                                        uint8_t* __restrict__ codes,
                                                        typename UxDt<DT>::T* __restrict__ scales,
                                                        uint8_t* __restrict__ zeros) {
  constexpr int LG = G / 8;
  const float qmax = (float)((1 << nbits) - 1);
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
    float x[8];
    load8_at<DT>(W, ldw, u * 8, kdiv, x);
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      mn = fminf(mn, x[i]);
      mx = fmaxf(mx, x[i]);
    }
    const UxQP q = ux_qparams<DT>(lanes_min<LG>(mn), lanes_max<LG>(mx), qmax);
    uint32_t c[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i >> 2] |= ux_code<DT>(x[i], q, qmax) << (8 * (i & 3));
    *reinterpret_cast<uint2*>(codes + (size_t)u * 8) = make_uint2(c[0], c[1]);
    if (u % LG == 0) {
      scales[u / LG] = UxDt<DT>::word(q.s);
      zeros[u / LG] = (uint8_t)q.zp;
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
      const uint32_t idx = j * L + i;
      if (idx < numel) v |= ((codes[idx] >> off) & ((1u << k) - 1u)) << (j * k);
    }
    shard[i] = (uint8_t)v;
  }
}

__device__ __forceinline__ uint32_t uintx_gather(const uint8_t* packed, const RaggedShards& sh, uint32_t numel,
                                                 uint32_t idx) {
  uint32_t c = 0;
  if (sh.has4) {
    const uint32_t L = (numel + 1) / 2;
    c |= (packed[sh.base4 + idx % L] >> (4 * (idx / L))) & 0xFu;
  }
  if (sh.has2) {
    const uint32_t L = (numel + 3) / 4;
    c |= ((packed[sh.base2 + idx % L] >> (2 * (idx / L))) & 0x3u) << sh.off2;
  }
  if (sh.has1) {
    const uint32_t L = (numel + 7) / 8;
    c |= ((packed[sh.base1 + idx % L] >> (idx / L)) & 0x1u) << sh.off1;
  }
  return c;
}

// Store 8 values that are already of the output dtype.
__device__ __forceinline__ void store8_f16(uint16_t* p, const float* d) {
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    w[q] = (uint32_t)UxDt<kF16>::word(d[2 * q]) | ((uint32_t)UxDt<kF16>::word(d[2 * q + 1]) << 16);
  st16_nt(p, U4{w[0], w[1], w[2], w[3]});
}

// Dequantize (SINK kStore: out of OUT = kF32 or the weight dtype) or accumulate the
// reconstruction error against W (SINK kErr), 8 consecutive elements per lane.
template <int DT, int G, int SINK, int OUT>
__global__ __launch_bounds__(256) void uintx_dequant_flat(const uint8_t* __restrict__ packed,
                                                          const typename UxDt<DT>::T* __restrict__ scales,
                                                          const uint8_t* __restrict__ zeros, FastDiv kdiv,
                                                          uint32_t units, uint32_t numel, RaggedShards sh,
                                                          void* __restrict__ out, int64_t ldo,
                                                          const typename UxDt<DT>::T* __restrict__ W, int64_t ldw,
                                                          double* __restrict__ part) {
  const uint32_t stride = gridDim.x * blockDim.x;
  double sw = 0.0, se = 0.0;
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
    const uint32_t e = u * 8;
    const float s = UxDt<DT>::value(scales[e / G]);
    const float zp = (float)zeros[e / G];
    float d[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = ux_value<DT>(uintx_gather(packed, sh, numel, e + i), zp, s);
    const uint32_t n = fdiv(e, kdiv);
    const uint32_t k = e - n * kdiv.d;
    if constexpr (SINK == kStore) {
      if constexpr (OUT == kF32) store8((float*)out + (int64_t)n * ldo + k, d);
      else if constexpr (OUT == kBF16) store8((uint16_t*)out + (int64_t)n * ldo + k, d);   // exact: d is bf16
      else store8_f16((uint16_t*)out + (int64_t)n * ldo + k, d);
    } else {
      float x[8];
      load8_dt<DT>(W + (int64_t)n * ldw + k, x);
      acc_err8(x, d, sw, se);
    }
  }
  if constexpr (SINK == kErr) block_sum2_store<256>(sw, se, part);
}

// ------------------------------------------------------------------ launchers
static unsigned capped_grid(uint64_t blocks, unsigned cap) {
  return (unsigned)(blocks < cap ? (blocks ? blocks : 1) : cap);
}

template <int DT, int G>
static void quant_flat_t(int nbits, const void* W, int64_t N, int64_t K, int64_t ldw, void* packed, void* scales,
                         void* zeros, void* workspace, hipStream_t st) {
  using T = typename UxDt<DT>::T;
  const uint32_t numel = (uint32_t)(N * K);
  const uint32_t units = numel / 8;
  uint8_t* codes = (uint8_t*)workspace;
  hipLaunchKernelGGL((uintx_codes_flat<DT, G>), dim3(capped_grid((units + 255) / 256, kStreamGridCap)), dim3(256),
                     0, st, (const T*)W, ldw, make_fastdiv((uint32_t)K), units, nbits, codes, (T*)scales,
                     (uint8_t*)zeros);
  const RaggedShards sh = ragged_shards(nbits, numel);
  int off = 0;
  for (int k : {4, 2, 1}) {
    if (!(nbits & k)) continue;
    const int64_t base = k == 4 ? sh.base4 : (k == 2 ? sh.base2 : sh.base1);
    const uint32_t L = (numel + (8 / k) - 1) / (8 / k);
    hipLaunchKernelGGL(uintx_pack_shard, dim3(capped_grid((L + 255) / 256, kStreamGridCap)), dim3(256), 0, st,
                       (const uint8_t*)codes, numel, k, off, (uint8_t*)packed + base);
    off += k;
  }
}

template <int DT, int G, int SINK, int OUT>
static void deq_flat_t(int nbits, const void* packed, const void* scales, const void* zeros, int64_t N, int64_t K,
                       void* out, int64_t ldo, const void* W, int64_t ldw, double* part, hipStream_t st) {
  using T = typename UxDt<DT>::T;
  const uint32_t numel = (uint32_t)(N * K);
  const unsigned grid = SINK == kErr ? uintx_flat_err_blocks(N, K)
                                     : capped_grid(((uint64_t)numel / 8 + 255) / 256, kStreamGridCap);
  hipLaunchKernelGGL((uintx_dequant_flat<DT, G, SINK, OUT>), dim3(grid), dim3(256), 0, st, (const uint8_t*)packed,
                     (const T*)scales, (const uint8_t*)zeros, make_fastdiv((uint32_t)K), numel / 8, numel,
                     ragged_shards(nbits, numel), out, ldo, (const T*)W, ldw, part);
}

// Dispatch over (dtype, group): the callers pass validated values only.
template <template <int, int> class F, typename... A>
static void by_dt_group(int32_t dt, int group, A... a) {
  if (dt == kBF16) {
    if (group == 32) F<kBF16, 32>::run(a...);
    else if (group == 64) F<kBF16, 64>::run(a...);
    else F<kBF16, 128>::run(a...);
  } else if (dt == kF16) {
    if (group == 32) F<kF16, 32>::run(a...);
    else if (group == 64) F<kF16, 64>::run(a...);
    else F<kF16, 128>::run(a...);
  } else {
    if (group == 32) F<kF32, 32>::run(a...);
    else if (group == 64) F<kF32, 64>::run(a...);
    else F<kF32, 128>::run(a...);
  }
}

template <int DT, int G> struct QuantFlat {
  static void run(int nbits, const void* W, int64_t N, int64_t K, int64_t ldw, void* packed, void* scales,
                  void* zeros, void* workspace, hipStream_t st) {
    quant_flat_t<DT, G>(nbits, W, N, K, ldw, packed, scales, zeros, workspace, st);
  }
};
template <int DT, int G> struct DeqFlat {
  static void run(int nbits, const void* packed, const void* scales, const void* zeros, int64_t N, int64_t K,
                  void* out, int32_t out_dtype, int64_t ldo, hipStream_t st) {
    if (out_dtype == kF32) deq_flat_t<DT, G, kStore, kF32>(nbits, packed, scales, zeros, N, K, out, ldo, nullptr, 0, nullptr, st);
    else deq_flat_t<DT, G, kStore, DT>(nbits, packed, scales, zeros, N, K, out, ldo, nullptr, 0, nullptr, st);
  }
};
template <int DT, int G> struct ErrFlat {
  static void run(int nbits, const void* W, int64_t N, int64_t K, int64_t ldw, const void* packed,
                  const void* scales, const void* zeros, double* part, hipStream_t st) {
    deq_flat_t<DT, G, kErr, kF32>(nbits, packed, scales, zeros, N, K, nullptr, 0, W, ldw, part, st);
  }
};

unsigned uintx_flat_err_blocks(int64_t N, int64_t K) {
  return capped_grid(((uint64_t)(N * K) / 8 + 255) / 256, kErrGridCap);
}

void launch_uintx_quant_flat(int nbits, int32_t dt, int group, const void* W, int64_t N, int64_t K, int64_t ldw,
                             void* packed, void* scales, void* zeros, void* workspace, hipStream_t st) {
  by_dt_group<QuantFlat>(dt, group, nbits, W, N, K, ldw, packed, scales, zeros, workspace, st);
}

void launch_uintx_dequant_flat(int nbits, int32_t dt, int group, const void* packed, const void* scales,
                               const void* zeros, int64_t N, int64_t K, void* out, int32_t out_dtype, int64_t ldo,
                               hipStream_t st) {
  by_dt_group<DeqFlat>(dt, group, nbits, packed, scales, zeros, N, K, out, out_dtype, ldo, st);
}

void launch_uintx_err_flat(int nbits, int32_t dt, int group, const void* W, int64_t N, int64_t K, int64_t ldw,
                           const void* packed, const void* scales, const void* zeros, double* part, hipStream_t st) {
  by_dt_group<ErrFlat>(dt, group, nbits, W, N, K, ldw, packed, scales, zeros, part, st);
}

}  // namespace gwb
