// OCP MXFP4 quantize+pack, unpack+dequantize and fused reconstruction error.
// Page quantize_dflash_mxfp4.py: the E2M1 table, quantize_mxfp4, dequantize_mxfp4.
//
// Work unit: 8 consecutive weights of one row (one 128-bit bf16 load). Four
// consecutive lanes hold one 32-weight block, so the block amax is two DPP steps.
// A unit's 8 codes are one 32-bit word of the packed output (byte j of the word =
// code(2j) | code(2j+1) << 4), so a wavefront stores 256 contiguous bytes.
#include "kernels.hpp"
#include "mxfp4_math.hpp"

namespace gwb {

template <typename TIn>
__global__ __launch_bounds__(256) void mxfp4_quant_kernel(const TIn* __restrict__ W, int64_t ldw,
                                                          uint32_t units, FastDiv upr,
                                                          uint32_t* __restrict__ packed,
                                                          uint8_t* __restrict__ e8m0) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
    uint32_t n = fdiv(u, upr);
    uint32_t kc = u - n * upr.d;
    float x[8];
    load8(W + (int64_t)n * ldw + 8 * kc, x);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = lanes_max<4>(amax);
    uint32_t e8 = mx_e8m0(amax);
    float inv = mx_inv_scale(e8);
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= e2m1_code(x[i], inv) << (4 * i);
    packed[u] = word;
    if ((u & 3u) == 0) e8m0[u >> 2] = (uint8_t)e8;
  }
}

// Unpack + dequantize. SINK == kStore writes out[n, k]; SINK == kErr reads W at the
// same place and accumulates sum w^2 and sum (w - d)^2 (float32 subtraction, float64
// sums) into per-block partials.
template <int SINK, typename TOut, typename TW>
__global__ __launch_bounds__(256) void mxfp4_dequant_kernel(const uint32_t* __restrict__ packed,
                                                            const uint8_t* __restrict__ e8m0,
                                                            uint32_t units, FastDiv upr,
                                                            TOut* __restrict__ out, int64_t ldo,
                                                            const TW* __restrict__ W, int64_t ldw,
                                                            double* __restrict__ part) {
  const uint32_t stride = gridDim.x * blockDim.x;
  double sw = 0.0, se = 0.0;
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
    uint32_t n = fdiv(u, upr);
    uint32_t kc = u - n * upr.d;
    uint32_t word = packed[u];
    float sc = mx_scale(e8m0[u >> 2]);
    float d[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = e2m1_value((word >> (4 * i)) & 0xFu, sc);
    if constexpr (SINK == kStore) {
      store8(out + (int64_t)n * ldo + 8 * kc, d);
    } else {
      float x[8];
      load8(W + (int64_t)n * ldw + 8 * kc, x);
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
static unsigned grid_for(uint64_t units, unsigned cap) {
  uint64_t g = (units + 255) / 256;
  return (unsigned)(g < cap ? (g ? g : 1) : cap);
}

void launch_mxfp4_quant(const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw,
                        void* packed, void* e8m0, hipStream_t st) {
  uint32_t units = (uint32_t)(N * K / 8);
  FastDiv upr = make_fastdiv((uint32_t)(K / 8));
  unsigned grid = grid_for(units, kStreamGridCap);
  if (w_dtype == kBF16)
    hipLaunchKernelGGL(mxfp4_quant_kernel<uint16_t>, dim3(grid), dim3(256), 0, st,
                       (const uint16_t*)W, ldw, units, upr, (uint32_t*)packed, (uint8_t*)e8m0);
  else
    hipLaunchKernelGGL(mxfp4_quant_kernel<float>, dim3(grid), dim3(256), 0, st,
                       (const float*)W, ldw, units, upr, (uint32_t*)packed, (uint8_t*)e8m0);
}

void launch_mxfp4_dequant(const void* packed, const void* e8m0, int64_t N, int64_t K, void* out,
                          int32_t out_dtype, int64_t ldo, hipStream_t st) {
  uint32_t units = (uint32_t)(N * K / 8);
  FastDiv upr = make_fastdiv((uint32_t)(K / 8));
  unsigned grid = grid_for(units, kStreamGridCap);
  if (out_dtype == kBF16)
    hipLaunchKernelGGL((mxfp4_dequant_kernel<kStore, uint16_t, uint16_t>), dim3(grid), dim3(256), 0, st,
                       (const uint32_t*)packed, (const uint8_t*)e8m0, units, upr, (uint16_t*)out, ldo,
                       (const uint16_t*)nullptr, (int64_t)0, (double*)nullptr);
  else
    hipLaunchKernelGGL((mxfp4_dequant_kernel<kStore, float, uint16_t>), dim3(grid), dim3(256), 0, st,
                       (const uint32_t*)packed, (const uint8_t*)e8m0, units, upr, (float*)out, ldo,
                       (const uint16_t*)nullptr, (int64_t)0, (double*)nullptr);
}

unsigned mxfp4_err_blocks(int64_t N, int64_t K) { return grid_for((uint64_t)(N * K / 8), kErrGridCap); }

void launch_mxfp4_err(const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw,
                      const void* packed, const void* e8m0, double* part, hipStream_t st) {
  uint32_t units = (uint32_t)(N * K / 8);
  FastDiv upr = make_fastdiv((uint32_t)(K / 8));
  unsigned grid = mxfp4_err_blocks(N, K);
  if (w_dtype == kBF16)
    hipLaunchKernelGGL((mxfp4_dequant_kernel<kErr, float, uint16_t>), dim3(grid), dim3(256), 0, st,
                       (const uint32_t*)packed, (const uint8_t*)e8m0, units, upr, (float*)nullptr,
                       (int64_t)0, (const uint16_t*)W, ldw, part);
  else
    hipLaunchKernelGGL((mxfp4_dequant_kernel<kErr, float, float>), dim3(grid), dim3(256), 0, st,
                       (const uint32_t*)packed, (const uint8_t*)e8m0, units, upr, (float*)nullptr,
                       (int64_t)0, (const float*)W, ldw, part);
}

}  // namespace gwb
