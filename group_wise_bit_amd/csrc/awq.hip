// AWQ-style alpha search on MXFP4. Page quantize_dflash_mxfp4.py, search_scale, with
// the diagonal surrogate of its module docstring: err(alpha) =
// sum(((dequant(quant_mxfp4(W * s)) / s - W) * a')**2), s a per-input-channel scaling.
//
// Kernel 1 (one block per alpha) builds that alpha's scaling row in float64 and rounds
// each entry once to float32: a' = max(a, 1e-8); an = a' / mean(a');
// s = clamp(an**alpha, 1e-2, 1e2); s /= exp(mean(log s)).
// Kernel 2 reads each weight of the row subsample once and evaluates every alpha in
// registers: X = W*s, the MXFP4 round trip of X (the same conversions as mxfp4.hip),
// D / s by IEEE division, then the weighted square in float32 and a float64 sum.
// Kernel 3 sums the per-block partials in a fixed order (one wavefront per alpha)
// and picks the first alpha with the strictly smallest error.
#include "kernels.hpp"
#include "mxfp4_math.hpp"

namespace gwb {

constexpr int kMaxAlpha = 16;
constexpr int kTableThreads = 1024;

struct Alphas {
  double v[kMaxAlpha];
};

template <int THREADS>
__device__ double block_sum(double v) {
  __shared__ double sh[THREADS];
  __syncthreads();
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int s = THREADS / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  return sh[0];
}

__device__ __forceinline__ double awq_s(double an, double alpha) {
  // exact special cases of an**alpha first (0 -> 1, 1 -> an, 0.5 -> correctly rounded sqrt)
  double p = alpha == 0.0 ? 1.0 : (alpha == 1.0 ? an : (alpha == 0.5 ? sqrt(an) : pow(an, alpha)));
  return fmin(fmax(p, 1e-2), 1e2);
}

__global__ __launch_bounds__(kTableThreads) void awq_table_kernel(const float* __restrict__ a, int K, Alphas al,
                                                                  float* __restrict__ table) {
  const double alpha = al.v[blockIdx.x];
  double acc = 0.0;
  for (int k = threadIdx.x; k < K; k += kTableThreads) acc += (double)fmaxf(a[k], 1e-8f);
  const double mean = block_sum<kTableThreads>(acc) / (double)K;
  double lg = 0.0;
  for (int k = threadIdx.x; k < K; k += kTableThreads) lg += log(awq_s((double)fmaxf(a[k], 1e-8f) / mean, alpha));
  const double g = exp(block_sum<kTableThreads>(lg) / (double)K);
  for (int k = threadIdx.x; k < K; k += kTableThreads)
    table[(int64_t)blockIdx.x * K + k] = (float)(awq_s((double)fmaxf(a[k], 1e-8f) / mean, alpha) / g);
}

template <typename TIn>
__global__ __launch_bounds__(256) void awq_search_kernel(const TIn* __restrict__ W, int64_t ldw, int64_t row_step,
                                                         uint32_t units, FastDiv upr, int K,
                                                         const float* __restrict__ a,
                                                         const float* __restrict__ table, int n_alpha,
                                                         double* __restrict__ part) {
  double acc[kMaxAlpha];
#pragma unroll
  for (int i = 0; i < kMaxAlpha; ++i) acc[i] = 0.0;
  const uint32_t stride = gridDim.x * blockDim.x;
  // units is a multiple of 4 and so is the stride: the 4 lanes of a block stay together
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
    const uint32_t r = fdiv(u, upr);
    const int k0 = 8 * (u - r * upr.d);
    float x[8], ap[8];
    to_f32(load_raw8(W + (int64_t)r * row_step * ldw + k0), x);
#pragma unroll
    for (int i = 0; i < 8; ++i) ap[i] = fmaxf(a[k0 + i], 1e-8f);
#pragma unroll
    for (int al = 0; al < kMaxAlpha; ++al) {
      if (al < n_alpha) {
        float s[8], X[8], D[8];
        load8(table + (int64_t)al * K + k0, s);
#pragma unroll
        for (int i = 0; i < 8; ++i) X[i] = x[i] * s[i];
        const uint32_t e8 = mx_e8m0_bits(quad_max_u(absmax8_bits(X)));
        mx_unpack8(mx_pack8(X, mx_scale_operand(e8)), e8, D);
        double sum = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float t = (D[i] / s[i] - x[i]) * ap[i];
          sum += (double)(t * t);
        }
        acc[al] += sum;
      }
    }
  }
#pragma unroll
  for (int al = 0; al < kMaxAlpha; ++al) {   // unrolled so acc stays in registers
    if (al < n_alpha) {
      const double v = block_sum<256>(acc[al]);
      if (threadIdx.x == 0) part[(int64_t)blockIdx.x * n_alpha + al] = v;
    }
  }
}

// One wavefront per alpha sums that alpha's partials (lane-strided, then a fixed
// butterfly), then thread 0 takes the first strict minimum.
__global__ __launch_bounds__(1024) void awq_finalize_kernel(const double* __restrict__ part, unsigned nblocks,
                                                            int n_alpha, double* __restrict__ err,
                                                            int32_t* __restrict__ best) {
  __shared__ double e[kMaxAlpha];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (wave < n_alpha) {
    double acc = 0.0;
    for (unsigned b = lane; b < nblocks; b += 64) acc += part[(int64_t)b * n_alpha + wave];
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) {
      e[wave] = acc;
      err[wave] = acc;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int bi = 0;
    for (int al = 1; al < n_alpha; ++al)
      if (e[al] < e[bi]) bi = al;
    best[0] = bi;
  }
}

unsigned awq_blocks(int64_t rows, int64_t K) { return err_blocks_for((uint64_t)(rows * K / 8)); }

void launch_awq(const void* W, int32_t w_dtype, int64_t rows, int64_t row_step, int64_t K, int64_t ldw,
                const float* a, const double* alphas, int n_alpha, float* s_table, double* err,
                int32_t* best, double* part, double* /*stat*/, hipStream_t st) {
  if (alphas) {
    Alphas al{};
    for (int i = 0; i < n_alpha; ++i) al.v[i] = alphas[i];
    hipLaunchKernelGGL(awq_table_kernel, dim3(n_alpha), dim3(kTableThreads), 0, st, a, (int)K, al, s_table);
  }
  const uint32_t units = (uint32_t)(rows * K / 8);
  const FastDiv upr = make_fastdiv((uint32_t)(K / 8));
  const unsigned grid = awq_blocks(rows, K);
  if (w_dtype == kBF16)
    hipLaunchKernelGGL(awq_search_kernel<uint16_t>, dim3(grid), dim3(256), 0, st, (const uint16_t*)W, ldw,
                       row_step, units, upr, (int)K, a, (const float*)s_table, n_alpha, part);
  else
    hipLaunchKernelGGL(awq_search_kernel<float>, dim3(grid), dim3(256), 0, st, (const float*)W, ldw, row_step,
                       units, upr, (int)K, a, (const float*)s_table, n_alpha, part);
  hipLaunchKernelGGL(awq_finalize_kernel, dim3(1), dim3(1024), 0, st, (const double*)part, grid, n_alpha, err, best);
}

}  // namespace gwb
