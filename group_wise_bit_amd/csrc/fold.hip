// Folding AWQ scales into weights, then requantizing to MXFP4, in one pass.
// Page quantize_dflash_mxfp4.py, main and its module docstring: after the alpha search
// the page divides the norm weights by s, multiplies the columns of the projections
// that read the normed input (and the conv's kernel projection) by s, divides up's
// rows by down's s, rounding each result to bfloat16, and then quantizes the folded
// weights with quantize_mxfp4.
//
// A fold here is an optional column step (multiply or divide by col[k]) followed by an
// optional row step (by row[n]), each one float32 operation rounded to bfloat16 (the
// hardware pair conversion, RNE); divisions are IEEE. The folded words can be stored
// (bf16, non-temporal) and/or quantized to MXFP4 exactly as mxfp4.hip does, so a
// folded linear that is served quantized never exists in HBM as bf16.
#include "kernels.hpp"
#include "mxfp4_math.hpp"

namespace gwb {

typedef __bf16 fd_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float fd_f32x2_t __attribute__((ext_vector_type(2)));

template <int OP>
__device__ __forceinline__ float fold_op(float x, float v) {
  if constexpr (OP == kFoldMul) return x * v;
  else return x / v;
}
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(fd_f32x2_t{a, b}, fd_bf16x2_t));
}

// One unit: 8 consecutive bf16 weights of row n from k0. Returns the folded bf16 words.
template <int COP, int ROP>
__device__ __forceinline__ U4 fold_unit(U4 w, const float* __restrict__ col, const float* __restrict__ row,
                                        uint32_t n, uint32_t k0) {
  if constexpr (COP != kFoldNone) {
    float x[8], c[8];
    to_f32(Raw8<uint16_t>{w}, x);
    load8(col + k0, c);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = fold_op<COP>(x[j], c[j]);
    w = U4{bf16_pair(x[0], x[1]), bf16_pair(x[2], x[3]), bf16_pair(x[4], x[5]), bf16_pair(x[6], x[7])};
  }
  if constexpr (ROP != kFoldNone) {
    const float r = row[n];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = bf16_pair(fold_op<ROP>(__uint_as_float(ws[q] << 16), r),
                       fold_op<ROP>(__uint_as_float(ws[q] & 0xFFFF0000u), r));
    w = U4{o[0], o[1], o[2], o[3]};
  }
  return w;
}

template <int COP, int ROP>
__device__ __forceinline__ void fold_store(U4 raw, uint32_t u, FastDiv upr,
                                           const float* __restrict__ col, const float* __restrict__ row,
                                           uint16_t* __restrict__ out, int64_t ldo,
                                           uint32_t* __restrict__ packed, uint8_t* __restrict__ e8m0) {
  const uint32_t n = fdiv(u, upr), k0 = 8 * (u - n * upr.d);
  const U4 w = fold_unit<COP, ROP>(raw, col, row, n, k0);
  if (out) st16_nt(out + (int64_t)n * ldo + k0, w);
  if (packed) {       // uniform per launch; the DPP step below has all four lanes
    const uint32_t e8 = mx_e8m0_bits(quad_max_u(absmax8_bits(w)));
    packed[u] = mx_pack8(w, mx_scale_operand(e8));
    if ((u & 3u) == 0) e8m0[u >> 2] = (uint8_t)e8;
  }
}

// Grid-stride over units of 8 weights, four loads in flight per lane. units = N*K/8 is
// a multiple of 4 and so is every stride, so the four lanes of a 32-block stay together.
template <int COP, int ROP>
__global__ __launch_bounds__(256) void fold_kernel(const uint16_t* __restrict__ W, int64_t ldw, uint32_t units,
                                                   FastDiv upr, const float* __restrict__ col,
                                                   const float* __restrict__ row, uint16_t* __restrict__ out,
                                                   int64_t ldo, uint32_t* __restrict__ packed,
                                                   uint8_t* __restrict__ e8m0) {
  const uint32_t stride = gridDim.x * blockDim.x;
  uint32_t u = blockIdx.x * blockDim.x + threadIdx.x;
  auto at = [&](uint32_t v) {
    const uint32_t n = fdiv(v, upr);
    return W + (int64_t)n * ldw + 8 * (v - n * upr.d);
  };
  for (; u + 3 * stride < units; u += 4 * stride) {
    const U4 r0 = ld16_nt(at(u)), r1 = ld16_nt(at(u + stride));
    const U4 r2 = ld16_nt(at(u + 2 * stride)), r3 = ld16_nt(at(u + 3 * stride));
    fold_store<COP, ROP>(r0, u, upr, col, row, out, ldo, packed, e8m0);
    fold_store<COP, ROP>(r1, u + stride, upr, col, row, out, ldo, packed, e8m0);
    fold_store<COP, ROP>(r2, u + 2 * stride, upr, col, row, out, ldo, packed, e8m0);
    fold_store<COP, ROP>(r3, u + 3 * stride, upr, col, row, out, ldo, packed, e8m0);
  }
  for (; u < units; u += stride) fold_store<COP, ROP>(ld16_nt(at(u)), u, upr, col, row, out, ldo, packed, e8m0);
}

// Column-fixed layout: when the grid stride S (in units of 8 weights) is a multiple of
// the units per row R = K/8, every unit of a lane sits at the same column offset k0 and
// the rows step by S / R: the lane loads its 8 column scales once, and no unit needs a
// division. Eight units' loads in flight per lane, grid-stride, as the MXFP4 quantize
// kernel (units % 4 == 0 and S % 4 == 0 keep the four lanes of a 32-block together).
template <int COP, int ROP>
__device__ __forceinline__ void fold_unit_fixk(U4 w, uint32_t u, uint32_t n, uint32_t k0, const float (&c)[8],
                                               const float* __restrict__ row, uint16_t* __restrict__ out,
                                               int64_t ldo, uint32_t* __restrict__ packed,
                                               uint8_t* __restrict__ e8m0) {
  if constexpr (COP != kFoldNone) {
    float x[8];
    to_f32(Raw8<uint16_t>{w}, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = fold_op<COP>(x[j], c[j]);
    w = U4{bf16_pair(x[0], x[1]), bf16_pair(x[2], x[3]), bf16_pair(x[4], x[5]), bf16_pair(x[6], x[7])};
  }
  if constexpr (ROP != kFoldNone) {
    const float r = row[n];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = bf16_pair(fold_op<ROP>(__uint_as_float(ws[q] << 16), r),
                       fold_op<ROP>(__uint_as_float(ws[q] & 0xFFFF0000u), r));
    w = U4{o[0], o[1], o[2], o[3]};
  }
  if (out) st16_nt(out + (int64_t)n * ldo + k0, w);
  if (packed) {       // uniform per launch; the DPP step below has all four lanes
    const uint32_t e8 = mx_e8m0_bits(quad_max_u(absmax8_bits(w)));
    // non-temporal, as the MXFP4 quantize kernel's codes; E8M0 bytes stay ordinary stores
    __builtin_nontemporal_store(mx_pack8(w, mx_scale_operand(e8)), packed + u);
    if ((u & 3u) == 0) e8m0[u >> 2] = (uint8_t)e8;
  }
}

template <int COP, int ROP>
__global__ __launch_bounds__(256) void fold_kernel_fixk(const uint16_t* __restrict__ W, int64_t ldw, uint32_t units,
                                                        uint32_t R, const float* __restrict__ col,
                                                        const float* __restrict__ row, uint16_t* __restrict__ out,
                                                        int64_t ldo, uint32_t* __restrict__ packed,
                                                        uint8_t* __restrict__ e8m0) {
  constexpr int U = 8;
  const uint32_t S = gridDim.x * blockDim.x, dn = S / R;
  uint32_t u = blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= units) return;                      // whole quads: units % 4 == 0
  uint32_t n = u / R;
  const uint32_t k0 = 8 * (u - n * R);
  float c[8] = {};
  if constexpr (COP != kFoldNone) load8(col + k0, c);
  for (; u + (U - 1) * S < units; u += U * S, n += U * dn) {
    U4 r[U];
#pragma unroll
    for (int i = 0; i < U; ++i) r[i] = ld16_nt(W + (int64_t)(n + i * dn) * ldw + k0);
#pragma unroll
    for (int i = 0; i < U; ++i)
      fold_unit_fixk<COP, ROP>(r[i], u + i * S, n + i * dn, k0, c, row, out, ldo, packed, e8m0);
  }
  for (; u < units; u += S, n += dn)
    fold_unit_fixk<COP, ROP>(ld16_nt(W + (int64_t)n * ldw + k0), u, n, k0, c, row, out, ldo, packed, e8m0);
}

// ------------------------------------------------------------------ launchers
// Resident blocks per compute unit of the column-fixed kernel, measured cold at the
// gate_up shape: 8 when only MXFP4 is written (1, 2, 4, 6, 8, 12, 16: 124, 93, 88, 85,
// 82, 85, 83 us), 1 when the folded bf16 weight is written too (1, 2, 4: 150, 163, 162 us).
constexpr int kFoldMxPerCU = 8, kFoldBf16PerCU = 1;
// Grid of the column-fixed kernel: about per_cu blocks per compute unit, a multiple of
// R / gcd(R, 256) so that the stride is whole rows; 0 when no such grid is near that.
static unsigned fixk_grid(uint32_t R, uint32_t units, int per_cu) {
  uint32_t g = R, b = 256;
  while (b) { const uint32_t t = g % b; g = b; b = t; }
  const uint32_t m = R / g;                    // blocks per whole-row stride
  const uint32_t target = stream_grid(units, per_cu);
  if (m > target) return 0;
  return target / m * m;
}

template <int COP, int ROP>
static void fold_launch_t(const void* W, int64_t N, int64_t K, int64_t ldw, const float* col, const float* row,
                          void* out, int64_t ldo, void* packed, void* e8m0, hipStream_t st) {
  const uint32_t units = (uint32_t)(N * K / 8);
  if (const unsigned g = fixk_grid((uint32_t)(K / 8), units, out ? kFoldBf16PerCU : kFoldMxPerCU)) {
    hipLaunchKernelGGL((fold_kernel_fixk<COP, ROP>), dim3(g), dim3(256), 0, st, (const uint16_t*)W, ldw, units,
                       (uint32_t)(K / 8), col, row, (uint16_t*)out, ldo, (uint32_t*)packed, (uint8_t*)e8m0);
    return;
  }
  const FastDiv upr = make_fastdiv((uint32_t)(K / 8));
  hipLaunchKernelGGL((fold_kernel<COP, ROP>), dim3(stream_blocks(units)), dim3(256), 0, st, (const uint16_t*)W, ldw,
                     units, upr, col, row, (uint16_t*)out, ldo, (uint32_t*)packed, (uint8_t*)e8m0);
}

template <int COP>
static void fold_launch_c(int row_op, const void* W, int64_t N, int64_t K, int64_t ldw,
                          const float* col, const float* row, void* out, int64_t ldo, void* packed, void* e8m0,
                          hipStream_t st) {
  if (row_op == kFoldMul) fold_launch_t<COP, kFoldMul>(W, N, K, ldw, col, row, out, ldo, packed, e8m0, st);
  else if (row_op == kFoldDiv) fold_launch_t<COP, kFoldDiv>(W, N, K, ldw, col, row, out, ldo, packed, e8m0, st);
  else fold_launch_t<COP, kFoldNone>(W, N, K, ldw, col, row, out, ldo, packed, e8m0, st);
}

void launch_fold(int col_op, int row_op, const void* W, int64_t N, int64_t K, int64_t ldw,
                 const float* col, const float* row, void* out, int64_t ldo, void* packed, void* e8m0,
                 hipStream_t st) {
  if (col_op == kFoldMul) fold_launch_c<kFoldMul>(row_op, W, N, K, ldw, col, row, out, ldo, packed, e8m0, st);
  else if (col_op == kFoldDiv) fold_launch_c<kFoldDiv>(row_op, W, N, K, ldw, col, row, out, ldo, packed, e8m0, st);
  else fold_launch_c<kFoldNone>(row_op, W, N, K, ldw, col, row, out, ldo, packed, e8m0, st);
}

}  // namespace gwb
