// AWQ-style alpha search on MXFP4. Page quantize_dflash_mxfp4.py, search_scale, with
// the diagonal surrogate of its module docstring: err(alpha) =
// sum(((dequant(quant_mxfp4(W * s)) / s - W) * a')**2), s a per-input-channel scaling.
//
// Kernel 1 (one block) builds the scaling table in float64 and rounds each entry once
// to float32: a' = max(a, 1e-8); an = a' / mean(a'); s = clamp(an**alpha, 1e-2, 1e2);
// s /= exp(mean(log s)).
// Kernel 2 reads each weight of the row subsample once and evaluates every alpha in
// registers: X = W*s, MXFP4 round trip of X (same arithmetic as mxfp4.hip), D / s by
// IEEE division, then the weighted square in float32 and a float64 running sum.
// Kernel 3 sums the per-block partials in a fixed order and picks the first alpha
// with the strictly smallest error.
#include "kernels.hpp"
#include "mxfp4_math.hpp"

namespace gwb {

constexpr int kMaxAlpha = 16;

struct Alphas {
  double v[kMaxAlpha];
};

__device__ double block_sum(double v) {
  __shared__ double sh[256];
  __syncthreads();
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
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

__global__ __launch_bounds__(256) void awq_table_kernel(const float* __restrict__ a, int K, Alphas al,
                                                        int n_alpha, float* __restrict__ table) {
  double acc = 0.0;
  for (int k = threadIdx.x; k < K; k += 256) acc += (double)fmaxf(a[k], 1e-8f);
  const double mean = block_sum(acc) / (double)K;
  for (int i = 0; i < n_alpha; ++i) {
    double lg = 0.0;
    for (int k = threadIdx.x; k < K; k += 256) lg += log(awq_s((double)fmaxf(a[k], 1e-8f) / mean, al.v[i]));
    const double g = exp(block_sum(lg) / (double)K);
    for (int k = threadIdx.x; k < K; k += 256)
      table[(int64_t)i * K + k] = (float)(awq_s((double)fmaxf(a[k], 1e-8f) / mean, al.v[i]) / g);
  }
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
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
    const uint32_t r = fdiv(u, upr);
    const uint32_t kc = u - r * upr.d;
    const int k0 = 8 * kc;
    float x[8], ap[8];
    load8(W + (int64_t)r * row_step * ldw + k0, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) ap[i] = fmaxf(a[k0 + i], 1e-8f);
#pragma unroll
    for (int al = 0; al < kMaxAlpha; ++al) {
      if (al < n_alpha) {
        float s[8], X[8];
        load8(table + (int64_t)al * K + k0, s);
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          X[i] = x[i] * s[i];
          amax = fmaxf(amax, fabsf(X[i]));
        }
        amax = lanes_max<4>(amax);
        const uint32_t e8 = mx_e8m0(amax);
        const float inv = mx_inv_scale(e8);
        const float sc = mx_scale(e8);
        double sum = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // D = +-r * 2**e with the sign of X (a negative that rounds to 0 gives -0.0)
          float r = e2m1_round_mag(X[i] * inv);
          float D = __uint_as_float(__float_as_uint(r * sc) | (__float_as_uint(X[i]) & 0x80000000u));
          float t = (D / s[i] - x[i]) * ap[i];
          sum += (double)(t * t);
        }
        acc[al] += sum;
      }
    }
  }
#pragma unroll
  for (int al = 0; al < kMaxAlpha; ++al) {   // unrolled so acc stays in registers
    if (al < n_alpha) {
      double v = block_sum(acc[al]);
      if (threadIdx.x == 0) part[(int64_t)blockIdx.x * n_alpha + al] = v;
    }
  }
}

__global__ __launch_bounds__(256) void awq_finalize_kernel(const double* __restrict__ part, unsigned nblocks,
                                                           int n_alpha, double* __restrict__ err,
                                                           int32_t* __restrict__ best) {
  __shared__ double e[kMaxAlpha];
  for (int al = 0; al < n_alpha; ++al) {
    double acc = 0.0;
    for (unsigned b = threadIdx.x; b < nblocks; b += 256) acc += part[(int64_t)b * n_alpha + al];
    double v = block_sum(acc);
    if (threadIdx.x == 0) {
      e[al] = v;
      err[al] = v;
    }
  }
  if (threadIdx.x == 0) {
    int bi = 0;
    for (int al = 1; al < n_alpha; ++al)
      if (e[al] < e[bi]) bi = al;
    best[0] = bi;
  }
}

unsigned awq_blocks(int64_t rows, int64_t K) {
  uint64_t units = (uint64_t)(rows * K / 8);
  uint64_t g = (units + 255) / 256;
  return (unsigned)(g < 2048 ? (g ? g : 1) : 2048);
}

void launch_awq(const void* W, int32_t w_dtype, int64_t rows, int64_t row_step, int64_t K, int64_t ldw,
                const float* a, const double* alphas, int n_alpha, float* s_table, double* err,
                int32_t* best, double* part, double* /*stat*/, hipStream_t st) {
  if (alphas) {
    Alphas al{};
    for (int i = 0; i < n_alpha; ++i) al.v[i] = alphas[i];
    hipLaunchKernelGGL(awq_table_kernel, dim3(1), dim3(256), 0, st, a, (int)K, al, n_alpha, s_table);
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
  hipLaunchKernelGGL(awq_finalize_kernel, dim3(1), dim3(256), 0, st, (const double*)part, grid, n_alpha, err, best);
}

}  // namespace gwb
