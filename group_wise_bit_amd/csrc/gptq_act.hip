// GPTQ with act-order groups (desc_act): the groups are formed over the input channels
// taken in a caller-given order, qweight stays in channel order and g_idx[k] names the
// group of channel k. Page export_gptq_cpu.py stores g_idx and writes desc_act into the
// checkpoint config; its per-group formulas (quantize_sym / quantize_asym) are used
// unchanged on those groups, and a consumer reads channel k with the scale and zero
// point of group g_idx[k].
//
// Quantization: (1) from the order perm, inv[perm[j]] = j and g_idx[perm[j]] = j / G;
// (2) gather the weight's columns into that order (a workspace copy); (3) the GPTQ
// quantize kernels on the copy, whose groups are then exactly the act-order groups and
// whose scales and zero points are final; (4) repack the codes back to channel order.
// Dequantization and the fused error: the tile kernel of gptq.hip with each channel's
// group read from g_idx; the tile's 32 rows of every group's scale (and zero point) sit
// in LDS, so K / G is limited to kActMaxGroups.
//
// perm must be a permutation of 0..K-1 and g_idx values must lie in [0, K/G): other
// values are clamped into range (no access leaves its buffer) and give unspecified codes.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gwb {

namespace {
constexpr int kTN = 32, kTK = 512, kTR = kTK / 8;   // the gptq.hip tile
constexpr int kQS = kTN + 1;

__device__ __forceinline__ uint32_t clamp_idx(int32_t v, uint32_t n) {
  return v < 0 ? 0u : ((uint32_t)v >= n ? n - 1 : (uint32_t)v);
}
}  // namespace

// inv[perm[j]] = j, g_idx[perm[j]] = j / G
__global__ __launch_bounds__(256) void act_order_index_kernel(const int32_t* __restrict__ perm, uint32_t K, int G,
                                                              int32_t* __restrict__ inv, int32_t* __restrict__ g_idx) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t j = blockIdx.x * blockDim.x + threadIdx.x; j < K; j += stride) {
    const uint32_t p = clamp_idx(perm[j], K);
    inv[p] = (int32_t)j;
    g_idx[p] = (int32_t)(j / (uint32_t)G);
  }
}

// Wp[n, j] = W[n, perm[j]], 8 consecutive j per thread (coalesced stores; the gathered
// loads stay within one row, which the L2 holds after its first touch).
template <typename T>
__global__ __launch_bounds__(256) void act_order_gather_kernel(const T* __restrict__ W, int64_t ldw,
                                                               const int32_t* __restrict__ perm, uint32_t K,
                                                               FastDiv upr, uint32_t units, T* __restrict__ Wp) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
    const uint32_t n = fdiv(u, upr), j0 = 8 * (u - n * upr.d);
    const T* row = W + (int64_t)n * ldw;
    T v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = row[clamp_idx(perm[j0 + i], K)];
    T* dst = Wp + (int64_t)n * K + j0;
    if constexpr (sizeof(T) == 2) {
      st16(dst, U4{(uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16),
                   (uint32_t)v[4] | ((uint32_t)v[5] << 16), (uint32_t)v[6] | ((uint32_t)v[7] << 16)});
    } else {
      st16(dst, U4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
      st16(dst + 4, U4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])});
    }
  }
}

// qweight[r, n] nibble i = code of channel 8r + i, read from the permuted codes at
// position inv[8r + i].
__global__ __launch_bounds__(256) void act_order_repack_kernel(const uint32_t* __restrict__ qweight_p,
                                                               const int32_t* __restrict__ inv, uint32_t K,
                                                               uint32_t N, uint32_t words,
                                                               uint32_t* __restrict__ qweight) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < words; u += stride) {
    const uint32_t r = u / N, n = u - r * N;
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t j = clamp_idx(inv[8 * r + i], K);
      w |= ((qweight_p[(int64_t)(j / 8) * N + n] >> (4 * (j % 8))) & 0xFu) << (4 * i);
    }
    qweight[u] = w;
  }
}

// Dequantize (SINK kStore) or accumulate the error against W (SINK kErr) with per-channel
// groups. The tile layout follows gptq_dequant_kernel: wave w holds rows 8w..8w+7 of the
// 32-row tile, lane l holds k = k0 + 8l..8l+7. LDS: the qweight tile, then the 32 rows
// of every group's fp16 scale bits, then (asymmetric) the 4 qzeros words of every group.
template <int SINK, bool SYM, typename TOut, typename TW>
__global__ __launch_bounds__(256) void gptq_act_dequant_kernel(const uint32_t* __restrict__ qweight,
                                                               const _Float16* __restrict__ scales,
                                                               const uint32_t* __restrict__ qzeros,
                                                               const int32_t* __restrict__ g_idx, int N, int K,
                                                               int NG, int ntk, int ntiles, TOut* __restrict__ out,
                                                               int64_t ldo, const TW* __restrict__ W, int64_t ldw,
                                                               double* __restrict__ part) {
  extern __shared__ uint32_t lds[];
  uint32_t* qtile = lds;                                            // [kTR][kQS]
  uint16_t* stile = reinterpret_cast<uint16_t*>(lds + kTR * kQS);   // [NG][kTN]
  uint32_t* ztile = lds + kTR * kQS + (NG * kTN + 1) / 2;           // [NG][kTN / 8]
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const uint16_t* scale_bits = reinterpret_cast<const uint16_t*>(scales);
  double sw = 0.0, se = 0.0;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int nt = tile / ntk, kt = tile - nt * ntk;
    const int n0 = nt * kTN, k0 = kt * kTK;
    const int r = t >> 2, c8 = (t & 3) * 8;
    const bool qok = k0 / 8 + r < K / 8 && n0 + c8 < N;
    U4 qa{}, qb{};
    if (qok) {
      const uint32_t* src = qweight + (int64_t)(k0 / 8 + r) * N + n0 + c8;
      qa = ld16(src);
      qb = ld16(src + 4);
    }
    const int k = k0 + lane * 8;
    uint32_t gi[8];
    if (k < K) {
      const U4 ga = ld16(g_idx + k), gb = ld16(g_idx + k + 4);
      const uint32_t g8[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) gi[j] = clamp_idx((int32_t)g8[j], (uint32_t)NG);
    }
    Raw8<TW> wr[8];
    if constexpr (SINK == kErr) {
      const int kc = min(k, K - 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) wr[i] = load_raw8(W + (int64_t)min(n0 + wave * 8 + i, N - 1) * ldw + kc);
    }
    for (int e = t; e < NG * kTN; e += 256) {
      const int g = e / kTN, rl = e - g * kTN;
      stile[e] = n0 + rl < N ? scale_bits[(int64_t)g * N + n0 + rl] : (uint16_t)0;
    }
    if constexpr (!SYM) {
      for (int e = t; e < NG * (kTN / 8); e += 256) {
        const int g = e / (kTN / 8), q = e - g * (kTN / 8);
        ztile[e] = n0 + 8 * q < N ? qzeros[(int64_t)g * (N / 8) + n0 / 8 + q] : 0u;
      }
    }
    if (qok) {
      uint32_t* dst = &qtile[r * kQS + c8];
      dst[0] = qa.x; dst[1] = qa.y; dst[2] = qa.z; dst[3] = qa.w;
      dst[4] = qb.x; dst[5] = qb.y; dst[6] = qb.z; dst[7] = qb.w;
    }
    __syncthreads();
    if (k < K) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rl = wave * 8 + i;
        const int n = n0 + rl;
        if (n < N) {
          const uint32_t word = qtile[lane * kQS + rl];
          float d[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float s = (float)__builtin_bit_cast(_Float16, stile[gi[j] * kTN + rl]);
            float z = 8.0f;
            if constexpr (!SYM) z = (float)((ztile[gi[j] * (kTN / 8) + rl / 8] >> (4 * (rl % 8))) & 0xFu);
            // (c - z) * s: the page's float ops; exact in float32 for a finite fp16 scale
            d[j] = ((float)((word >> (4 * j)) & 0xFu) - z) * s;
          }
          if constexpr (SINK == kStore) {
            store8(out + (int64_t)n * ldo + k, d);
          } else {
            float x[8];
            to_f32(wr[i], x);
            acc_err8(x, d, sw, se);
          }
        }
      }
    }
    __syncthreads();
  }
  if constexpr (SINK == kErr) block_sum2_store<256>(sw, se, part);
}

// ------------------------------------------------------------------ launchers
static int act_ntk(int64_t K) { return (int)((K + kTK - 1) / kTK); }
static unsigned act_tiles(int64_t N, int64_t K) { return (unsigned)(((N + kTN - 1) / kTN) * act_ntk(K)); }
static size_t act_lds_bytes(bool sym, int NG) {
  return sizeof(uint32_t) * ((size_t)kTR * kQS + ((size_t)NG * kTN + 1) / 2 + (sym ? 0 : (size_t)NG * (kTN / 8)));
}
static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t gptq_act_workspace_bytes(int32_t w_dtype, int64_t N, int64_t K) {
  const size_t esize = w_dtype == kF32 ? 4 : 2;
  return align256((size_t)(N * K) * esize) + align256((size_t)(K / 8 * N) * 4) + align256((size_t)K * 4);
}

void launch_gptq_act_quant(bool sym, int group, const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw,
                           const int32_t* perm, void* qweight, void* scales, void* qzeros, int32_t* g_idx,
                           void* workspace, hipStream_t st) {
  const size_t esize = w_dtype == kF32 ? 4 : 2;
  uint8_t* ws = (uint8_t*)workspace;
  void* Wp = ws;
  uint32_t* qweight_p = (uint32_t*)(ws + align256((size_t)(N * K) * esize));
  int32_t* inv = (int32_t*)((uint8_t*)qweight_p + align256((size_t)(K / 8 * N) * 4));
  hipLaunchKernelGGL(act_order_index_kernel, dim3(stream_blocks((uint64_t)K)), dim3(256), 0, st, perm, (uint32_t)K,
                     group, inv, g_idx);
  const uint32_t units = (uint32_t)(N * K / 8);
  const FastDiv upr = make_fastdiv((uint32_t)(K / 8));
  if (w_dtype == kBF16)
    hipLaunchKernelGGL((act_order_gather_kernel<uint16_t>), dim3(stream_blocks(units)), dim3(256), 0, st,
                       (const uint16_t*)W, ldw, perm, (uint32_t)K, upr, units, (uint16_t*)Wp);
  else
    hipLaunchKernelGGL((act_order_gather_kernel<float>), dim3(stream_blocks(units)), dim3(256), 0, st,
                       (const float*)W, ldw, perm, (uint32_t)K, upr, units, (float*)Wp);
  launch_gptq_quant(sym, group, Wp, w_dtype, N, K, K, qweight_p, scales, qzeros, nullptr, st);
  const uint32_t words = (uint32_t)(K / 8 * N);
  hipLaunchKernelGGL(act_order_repack_kernel, dim3(stream_blocks(words)), dim3(256), 0, st,
                     (const uint32_t*)qweight_p, (const int32_t*)inv, (uint32_t)K, (uint32_t)N, words,
                     (uint32_t*)qweight);
}

template <int SINK, bool SYM, typename TOut, typename TW>
static void act_deq_launch(unsigned grid, int group, const void* qw, const void* sc, const void* qz,
                           const int32_t* g_idx, int64_t N, int64_t K, void* out, int64_t ldo, const void* W,
                           int64_t ldw, double* part, hipStream_t st) {
  const int NG = (int)(K / group);
  hipLaunchKernelGGL((gptq_act_dequant_kernel<SINK, SYM, TOut, TW>), dim3(grid), dim3(256), act_lds_bytes(SYM, NG),
                     st, (const uint32_t*)qw, (const _Float16*)sc, (const uint32_t*)qz, g_idx, (int)N, (int)K, NG,
                     act_ntk(K), (int)act_tiles(N, K), (TOut*)out, ldo, (const TW*)W, ldw, part);
}

void launch_gptq_act_dequant(bool sym, int group, const void* qweight, const void* scales, const void* qzeros,
                             const int32_t* g_idx, int64_t N, int64_t K, void* out, int32_t out_dtype, int64_t ldo,
                             hipStream_t st) {
  const unsigned grid = act_tiles(N, K);
  if (sym) {
    if (out_dtype == kBF16)
      act_deq_launch<kStore, true, uint16_t, uint16_t>(grid, group, qweight, scales, qzeros, g_idx, N, K, out, ldo,
                                                       nullptr, 0, nullptr, st);
    else
      act_deq_launch<kStore, true, float, uint16_t>(grid, group, qweight, scales, qzeros, g_idx, N, K, out, ldo,
                                                    nullptr, 0, nullptr, st);
  } else {
    if (out_dtype == kBF16)
      act_deq_launch<kStore, false, uint16_t, uint16_t>(grid, group, qweight, scales, qzeros, g_idx, N, K, out, ldo,
                                                        nullptr, 0, nullptr, st);
    else
      act_deq_launch<kStore, false, float, uint16_t>(grid, group, qweight, scales, qzeros, g_idx, N, K, out, ldo,
                                                     nullptr, 0, nullptr, st);
  }
}

unsigned gptq_act_err_blocks(int64_t N, int64_t K) {
  const unsigned t = act_tiles(N, K);
  const unsigned cap = 16 * kErrGridCap;
  return t < cap ? (t ? t : 1) : cap;
}

void launch_gptq_act_err(bool sym, int group, const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw,
                         const void* qweight, const void* scales, const void* qzeros, const int32_t* g_idx,
                         double* part, hipStream_t st) {
  const unsigned grid = gptq_act_err_blocks(N, K);
  if (sym) {
    if (w_dtype == kBF16)
      act_deq_launch<kErr, true, float, uint16_t>(grid, group, qweight, scales, qzeros, g_idx, N, K, nullptr, 0, W,
                                                  ldw, part, st);
    else
      act_deq_launch<kErr, true, float, float>(grid, group, qweight, scales, qzeros, g_idx, N, K, nullptr, 0, W, ldw,
                                               part, st);
  } else {
    if (w_dtype == kBF16)
      act_deq_launch<kErr, false, float, uint16_t>(grid, group, qweight, scales, qzeros, g_idx, N, K, nullptr, 0, W,
                                                   ldw, part, st);
    else
      act_deq_launch<kErr, false, float, float>(grid, group, qweight, scales, qzeros, g_idx, N, K, nullptr, 0, W,
                                                ldw, part, st);
  }
}

}  // namespace gwb
