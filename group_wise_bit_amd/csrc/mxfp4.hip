// OCP MXFP4 quantize+pack, unpack+dequantize and fused reconstruction error.
// Page quantize_dflash_mxfp4.py: the E2M1 table, quantize_mxfp4, dequantize_mxfp4.
//
// Work unit: 8 consecutive weights of one row (one 128-bit bf16 load). Four
// consecutive lanes hold one 32-weight block, so the block amax is two DPP steps. A
// unit's 8 codes are one 32-bit word of the packed output (byte j of the word =
// code(2j) | code(2j+1) << 4), so a wavefront stores 256 contiguous bytes. Each lane
// keeps four units' loads in flight before converting them (grid-stride, a few blocks
// per compute unit), which is what the HBM3E stream needs to stay busy.
#include "kernels.hpp"
#include "mxfp4_math.hpp"

namespace gwb {

// Launch shape of the streaming MXFP4 kernels (measured at the metric shape with inputs
// cold): units in flight per lane, resident blocks per compute unit of the quantize and
// dequantize passes, and the fixed block count of the error passes (whose partial sums
// the workspace holds, so it depends on the shape only).
constexpr int kMxUnits = 8;
constexpr int kMxQuantPerCU = 2;
constexpr int kMxDequantPerCU = 1;
constexpr unsigned kMxErrBlocks = 512;

__device__ __forceinline__ uint32_t absmax_bits(const Raw8<uint16_t>& r) { return absmax8_bits(r.v); }
__device__ __forceinline__ uint32_t absmax_bits(const Raw8<float>& r) {
  float x[8];
  to_f32(r, x);
  return absmax8_bits(x);
}
__device__ __forceinline__ uint32_t pack_unit(const Raw8<uint16_t>& r, float sc) { return mx_pack8(r.v, sc); }
__device__ __forceinline__ uint32_t pack_unit(const Raw8<float>& r, float sc) {
  float x[8];
  to_f32(r, x);
  return mx_pack8(x, sc);
}

// Address of unit u: rows of K/8 units, row stride ld elements. With contiguous rows
// (ld == K) the unit index is the element offset / 8 and no division is needed.
template <bool CONTIG, typename T>
__device__ __forceinline__ T* unit_ptr(T* base, int64_t ld, uint32_t u, FastDiv upr) {
  if constexpr (CONTIG) return base + (int64_t)u * 8;
  const uint32_t n = fdiv(u, upr);
  return base + (int64_t)n * ld + 8 * (u - n * upr.d);
}

// The page's own tie rule (its code takes the first tied index, then rounds that index
// down to even) differs from round-half-to-even at three magnitudes only: |x| / 2^e =
// 0.75, 1.75 and 3.5 go to codes 0, 2 and 4 instead of 2, 4 and 6. Returns what to
// subtract from the word (2 in each such nibble; the magnitude bits never borrow from
// the sign bit since the magnitude is at least 2).
template <typename TIn>
__device__ __forceinline__ uint32_t page_tie_fix(const Raw8<TIn>& r, uint32_t e8) {
  float x[8];
  to_f32(r, x);
  const int e = (int)e8 - 127;
  const float t1 = ldexpf(0.75f, e), t2 = ldexpf(1.75f, e), t3 = ldexpf(3.5f, e);
  uint32_t corr = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = fabsf(x[i]);
    if (a == t1 || a == t2 || a == t3) corr |= 2u << (4 * i);
  }
  return corr;
}

// SNR: also the reconstruction sums of the stored values (the dequantize kernel's
// arithmetic on the word and scale just written), in the error kernel's per-thread
// order when launched on its grid.
template <bool LIT, bool SNR, typename TIn>
__device__ __forceinline__ void quant_unit(const Raw8<TIn>& r, uint32_t u, uint32_t* __restrict__ packed,
                                           uint8_t* __restrict__ e8m0, double& sw, double& se) {
  const uint32_t e8 = mx_e8m0_bits(quad_max_u(absmax_bits(r)));
  uint32_t w = pack_unit(r, mx_scale_operand(e8));
  if constexpr (LIT) w -= page_tie_fix(r, e8);
  // non-temporal: the packed codes are read back much later, if at all, and ordinary
  // stores would leave them as dirty lines for the next kernel to write back (the small
  // E8M0 bytes stay ordinary stores, which L2 merges into lines)
  __builtin_nontemporal_store(w, packed + u);
  if ((u & 3u) == 0) e8m0[u >> 2] = (uint8_t)e8;
  if constexpr (SNR) {
    float d[8], x[8];
    mx_unpack8(w, e8, d);
    to_f32(r, x);
    // blocks whose maximum reaches 2^60 (E8M0 byte 185 or more) square in float64
    if (e8 >= 127u + 58u) acc_err8(x, d, sw, se);
    else if constexpr (sizeof(TIn) == 2) acc_err8_f32_bf16(r.v, x, d, sw, se);
    else acc_err8_f32(x, d, sw, se);
  }
}

// units = N*K/8 is a multiple of 4 and every stride is too, so the four lanes of a
// block always take the same branch of each loop (the DPP step needs all four). Each
// lane has kMxUnits units' loads in flight before converting them.
template <bool CONTIG, bool LIT, typename TIn, bool SNR>
__global__ __launch_bounds__(256) void mxfp4_quant_kernel(const TIn* __restrict__ W, int64_t ldw,
                                                          uint32_t units, FastDiv upr,
                                                          uint32_t* __restrict__ packed,
                                                          uint8_t* __restrict__ e8m0, double* __restrict__ part) {
  const uint32_t stride = gridDim.x * blockDim.x;
  double sw = 0.0, se = 0.0;
  uint32_t u = blockIdx.x * blockDim.x + threadIdx.x;
  for (; u + (kMxUnits - 1) * stride < units; u += kMxUnits * stride) {
    Raw8<TIn> r[kMxUnits];
#pragma unroll
    for (int i = 0; i < kMxUnits; ++i) r[i] = load_raw8(unit_ptr<CONTIG>(W, ldw, u + i * stride, upr));
#pragma unroll
    for (int i = 0; i < kMxUnits; ++i) quant_unit<LIT, SNR>(r[i], u + i * stride, packed, e8m0, sw, se);
  }
  for (; u < units; u += stride)
    quant_unit<LIT, SNR>(load_raw8(unit_ptr<CONTIG>(W, ldw, u, upr)), u, packed, e8m0, sw, se);
  if constexpr (SNR) block_sum2_store<256>(sw, se, part);
}

// Unpack + dequantize. SINK == kStore writes out[n, k]; SINK == kErr takes W at the
// same place (loaded by the caller with the packed word) and accumulates sum w^2 and
// sum (w - d)^2 into per-block partials.
template <int SINK, bool CONTIG, typename TOut, typename TW>
__device__ __forceinline__ void dequant_unit(uint32_t word, uint32_t e8, uint32_t u, FastDiv upr,
                                             TOut* __restrict__ out, int64_t ldo, const Raw8<TW>& wraw,
                                             double& sw, double& se) {
  if constexpr (SINK == kStore) {
    if constexpr (sizeof(TOut) == 2) {
      st16_nt(unit_ptr<CONTIG>(out, ldo, u, upr), mx_unpack8_bf16(word, e8));
    } else {
      float d[8];
      mx_unpack8(word, e8, d);
      store8(unit_ptr<CONTIG>(out, ldo, u, upr), d);
    }
  } else {
    float d[8], x[8];
    mx_unpack8(word, e8, d);
    to_f32(wraw, x);
    acc_err8(x, d, sw, se);
  }
}

template <int SINK, bool CONTIG, typename TOut, typename TW>
__global__ __launch_bounds__(256) void mxfp4_dequant_kernel(const uint32_t* __restrict__ packed,
                                                            const uint8_t* __restrict__ e8m0,
                                                            uint32_t units, FastDiv upr,
                                                            TOut* __restrict__ out, int64_t ldo,
                                                            const TW* __restrict__ W, int64_t ldw,
                                                            double* __restrict__ part) {
  const uint32_t stride = gridDim.x * blockDim.x;
  double sw = 0.0, se = 0.0;
  uint32_t u = blockIdx.x * blockDim.x + threadIdx.x;
  Raw8<TW> x[kMxUnits] = {};
  for (; u + (kMxUnits - 1) * stride < units; u += kMxUnits * stride) {
    uint32_t w[kMxUnits], e[kMxUnits];
#pragma unroll
    for (int i = 0; i < kMxUnits; ++i) {
      w[i] = ld4_nt(packed + u + i * stride);
      e[i] = e8m0[(u + i * stride) >> 2];
      if constexpr (SINK == kErr) x[i] = load_raw8(unit_ptr<CONTIG>(W, ldw, u + i * stride, upr));
    }
#pragma unroll
    for (int i = 0; i < kMxUnits; ++i)
      dequant_unit<SINK, CONTIG>(w[i], e[i], u + i * stride, upr, out, ldo, x[i], sw, se);
  }
  for (; u < units; u += stride) {
    if constexpr (SINK == kErr) x[0] = load_raw8(unit_ptr<CONTIG>(W, ldw, u, upr));
    dequant_unit<SINK, CONTIG>(packed[u], (uint32_t)e8m0[u >> 2], u, upr, out, ldo, x[0], sw, se);
  }
  if constexpr (SINK == kErr) block_sum2_store<256>(sw, se, part);
}

// ------------------------------------------------------------------ launchers
template <bool LIT, bool SNR>
static void quant_lit(const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw, void* packed, void* e8m0,
                      double* part, hipStream_t st) {
  const uint32_t units = (uint32_t)(N * K / 8);
  const FastDiv upr = make_fastdiv((uint32_t)(K / 8));
  // with the sums: the error kernel's grid, whose partials the workspace holds
  const unsigned grid = SNR ? mxfp4_err_blocks(N, K) : stream_grid(units, kMxQuantPerCU);
  const bool contig = ldw == K;
  if (w_dtype == kBF16)
    hipLaunchKernelGGL((contig ? mxfp4_quant_kernel<true, LIT, uint16_t, SNR>
                               : mxfp4_quant_kernel<false, LIT, uint16_t, SNR>),
                       dim3(grid), dim3(256), 0, st, (const uint16_t*)W, ldw, units, upr, (uint32_t*)packed,
                       (uint8_t*)e8m0, part);
  else
    hipLaunchKernelGGL((contig ? mxfp4_quant_kernel<true, LIT, float, SNR> : mxfp4_quant_kernel<false, LIT, float, SNR>),
                       dim3(grid), dim3(256), 0, st, (const float*)W, ldw, units, upr, (uint32_t*)packed,
                       (uint8_t*)e8m0, part);
}

void launch_mxfp4_quant(bool page_ties, const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw,
                        void* packed, void* e8m0, double* part, hipStream_t st) {
  if (page_ties) {
    if (part) quant_lit<true, true>(W, w_dtype, N, K, ldw, packed, e8m0, part, st);
    else quant_lit<true, false>(W, w_dtype, N, K, ldw, packed, e8m0, nullptr, st);
  } else {
    if (part) quant_lit<false, true>(W, w_dtype, N, K, ldw, packed, e8m0, part, st);
    else quant_lit<false, false>(W, w_dtype, N, K, ldw, packed, e8m0, nullptr, st);
  }
}

void launch_mxfp4_dequant(const void* packed, const void* e8m0, int64_t N, int64_t K, void* out,
                          int32_t out_dtype, int64_t ldo, hipStream_t st) {
  const uint32_t units = (uint32_t)(N * K / 8);
  const FastDiv upr = make_fastdiv((uint32_t)(K / 8));
  const unsigned grid = stream_grid(units, kMxDequantPerCU);
  const bool contig = ldo == K;
  if (out_dtype == kBF16)
    hipLaunchKernelGGL((contig ? mxfp4_dequant_kernel<kStore, true, uint16_t, uint16_t> : mxfp4_dequant_kernel<kStore, false, uint16_t, uint16_t>),
                       dim3(grid), dim3(256), 0, st, (const uint32_t*)packed, (const uint8_t*)e8m0, units, upr,
                       (uint16_t*)out, ldo, (const uint16_t*)nullptr, (int64_t)0, (double*)nullptr);
  else
    hipLaunchKernelGGL((contig ? mxfp4_dequant_kernel<kStore, true, float, uint16_t> : mxfp4_dequant_kernel<kStore, false, float, uint16_t>),
                       dim3(grid), dim3(256), 0, st, (const uint32_t*)packed, (const uint8_t*)e8m0, units, upr,
                       (float*)out, ldo, (const uint16_t*)nullptr, (int64_t)0, (double*)nullptr);
}

unsigned mxfp4_err_blocks(int64_t N, int64_t K) {
  const uint64_t g = ((uint64_t)(N * K / 8) + 255) / 256;
  return (unsigned)(g < kMxErrBlocks ? (g ? g : 1) : kMxErrBlocks);
}

void launch_mxfp4_err(const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw,
                      const void* packed, const void* e8m0, double* part, hipStream_t st) {
  const uint32_t units = (uint32_t)(N * K / 8);
  const FastDiv upr = make_fastdiv((uint32_t)(K / 8));
  const unsigned grid = mxfp4_err_blocks(N, K);
  const bool contig = ldw == K;
  if (w_dtype == kBF16)
    hipLaunchKernelGGL((contig ? mxfp4_dequant_kernel<kErr, true, float, uint16_t> : mxfp4_dequant_kernel<kErr, false, float, uint16_t>),
                       dim3(grid), dim3(256), 0, st, (const uint32_t*)packed, (const uint8_t*)e8m0, units, upr,
                       (float*)nullptr, (int64_t)0, (const uint16_t*)W, ldw, part);
  else
    hipLaunchKernelGGL((contig ? mxfp4_dequant_kernel<kErr, true, float, float> : mxfp4_dequant_kernel<kErr, false, float, float>),
                       dim3(grid), dim3(256), 0, st, (const uint32_t*)packed, (const uint8_t*)e8m0, units, upr,
                       (float*)nullptr, (int64_t)0, (const float*)W, ldw, part);
}

}  // namespace gwb
