// AWQ-style alpha search on MXFP4. Page quantize_dflash_mxfp4.py, search_scale, with
// the diagonal surrogate of its module docstring: err(alpha) =
// sum(((dequant(quant_mxfp4(W * s)) / s - W) * a')**2), s a per-input-channel scaling.
//
// Scalings, two kernels over (256-column chunk, alpha) blocks: a' = max(a, 1e-8);
// an = a' / mean(a'); p = clamp(an**alpha, 1e-2, 1e2) and each chunk's sum of log p in
// float64; then s = p / exp(mean(log p)) rounded once to float32, together with the
// float32 quotients 1/s and 1.5/s that the search uses.
// Search: a wavefront task is 4 subsample rows x 512 columns. A lane keeps 8 columns of
// its 4 rows in registers and evaluates every alpha on them: X = W*s, the MXFP4 round
// trip of X (the conversions of mxfp4.hip), D / s, the weighted square in float32 and
// a float64 sum. Per-block partials are summed in a fixed order, one wavefront per
// alpha, and the first alpha with the strictly smallest error wins.
//
// D / s without a division: a dequantized value is c * 2^E with c on the e2m1 grid
// {0, 0.5, 1, 1.5, 2, 3, 4, 6}, so D is +-2^m, +-1.5 * 2^m or +-0. With P the value D
// with its mantissa cleared (+-2^m or +-0), D / s = P * (1 / s) or P * (1.5 / s), and
// scaling a correctly rounded quotient by a power of two is exact while the product
// stays normal (or zero): fl(D / s) = P * fl(1 / s) or P * fl(1.5 / s). For s in
// [2^-14, 2^14] both quotients lie in [2^-14, 2^15); a block's nonzero codes have P in
// [2^(e8 - 128), 2^(e8 - 125)], so every product is normal when 16 <= e8 <= 238. Other
// blocks, and scalings outside that range (possible only in a caller's table), divide.
#include "kernels.hpp"
#include "mxfp4_math.hpp"

namespace gwb {

constexpr int kMaxAlpha = 16;
constexpr int kChunk = 256;                 // columns per block of the scaling kernels
constexpr int kRB = 4;                      // subsample rows a lane keeps
constexpr int kTaskCols = 512;              // columns of a wavefront task (64 lanes x 8)
constexpr int kTasksPerBlock = 4;           // one per wavefront
constexpr unsigned kSearchGridCap = 4096;
// Loads a thread issues before summing them in order: the table and partial reads come
// from the previous kernel's output in the Infinity Cache, and one round of loads instead
// of one per value keeps these small kernels from waiting on each load in turn.
constexpr int kLoadBatch = 32;

struct Alphas {
  double v[kMaxAlpha];
};

// Sum over the block, the same value in every thread: each wavefront's sum
// (wave_sum_f64), then the wavefront sums in order through LDS.
template <int THREADS>
__device__ double block_sum(double v) {
  __shared__ double sh[THREADS / 64];
  v = wave_sum_f64(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = sh[0];
#pragma unroll
  for (int i = 1; i < THREADS / 64; ++i) t += sh[i];
  return t;
}

__device__ __forceinline__ double awq_p(double an, double alpha) {
  // exact special cases of an**alpha first (0 -> 1, 1 -> an, 0.5 -> correctly rounded sqrt)
  double p = alpha == 0.0 ? 1.0 : (alpha == 1.0 ? an : (alpha == 0.5 ? sqrt(an) : pow(an, alpha)));
  return fmin(fmax(p, 1e-2), 1e2);
}

// grid (chunks, n_alpha): p for 256 columns of one alpha, and their sum of log p. Every
// block sums a' over all K in the same order, so all see the same mean.
__global__ __launch_bounds__(kChunk) void awq_pow_kernel(const float* __restrict__ a, int K, Alphas al,
                                                         double* __restrict__ pw, double* __restrict__ logs) {
  const int ai = blockIdx.y;
  double acc = 0.0;
  for (int base = 0; base < K; base += kChunk * kLoadBatch) {   // k = t, t + 256, ... in order
    float v[kLoadBatch];
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j) {
      const int k = base + j * kChunk + threadIdx.x;
      v[j] = a[min(k, K - 1)];                                    // loads without branches
    }
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j)
      if (base + j * kChunk + (int)threadIdx.x < K) acc += (double)fmaxf(v[j], 1e-8f);
  }
  const double mean = block_sum<kChunk>(acc) / (double)K;
  const int k = blockIdx.x * kChunk + threadIdx.x;
  double lg = 0.0;
  if (k < K) {
    const double p = awq_p((double)fmaxf(a[k], 1e-8f) / mean, al.v[ai]);
    pw[(int64_t)ai * K + k] = p;
    lg = log(p);
  }
  lg = block_sum<kChunk>(lg);
  if (threadIdx.x == 0) logs[(int64_t)ai * gridDim.x + blockIdx.x] = lg;
}

// grid (chunks, n_alpha): s = p / geomean(p) (pw != NULL), or the caller's s; then
// rc[alpha] = {1/s [K], 1.5/s [K]} in float32.
__global__ __launch_bounds__(kChunk) void awq_scale_kernel(const double* __restrict__ pw,
                                                           const double* __restrict__ logs, int K,
                                                           float* __restrict__ s_table, float* __restrict__ rc) {
  const int ai = blockIdx.y, k = blockIdx.x * kChunk + threadIdx.x;
  if (k >= K) return;
  float s;
  if (pw) {
    double lg = 0.0;
    for (unsigned c0 = 0; c0 < gridDim.x; c0 += kLoadBatch) {   // chunk order
      double v[kLoadBatch];
#pragma unroll
      for (int j = 0; j < kLoadBatch; ++j) v[j] = logs[(int64_t)ai * gridDim.x + min(c0 + j, gridDim.x - 1)];
#pragma unroll
      for (int j = 0; j < kLoadBatch; ++j)
        if (c0 + j < gridDim.x) lg += v[j];
    }
    s = (float)(pw[(int64_t)ai * K + k] / exp(lg / (double)K));
    s_table[(int64_t)ai * K + k] = s;
  } else {
    s = s_table[(int64_t)ai * K + k];
  }
  rc[(int64_t)ai * 2 * K + k] = 1.0f / s;
  rc[(int64_t)ai * 2 * K + K + k] = 1.5f / s;
}

template <typename TIn>
__global__ __launch_bounds__(256) void awq_search_kernel(const TIn* __restrict__ W, int64_t ldw, int64_t row_step,
                                                         int rows, int K, int nchunk, int ntasks,
                                                         const float* __restrict__ a,
                                                         const float* __restrict__ s_table,
                                                         const float* __restrict__ rc, int n_alpha,
                                                         double* __restrict__ part) {
  double acc[kMaxAlpha];
#pragma unroll
  for (int i = 0; i < kMaxAlpha; ++i) acc[i] = 0.0;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  for (int task = blockIdx.x * kTasksPerBlock + wave; task < ntasks; task += gridDim.x * kTasksPerBlock) {
    const int rb = task / nchunk, ch = task - rb * nchunk;
    const int k0 = ch * kTaskCols + lane * 8;
    // lanes past K (whole 32-blocks, K % 32 == 0) and rows past the subsample read a
    // valid place and add nothing
    const int kc = min(k0, K - 8);
    float x[kRB][8];
    bool use[kRB];
#pragma unroll
    for (int i = 0; i < kRB; ++i) {
      const int r = rb * kRB + i;
      use[i] = k0 < K && r < rows;
      to_f32(load_raw8(W + (int64_t)min(r, rows - 1) * row_step * ldw + kc), x[i]);
    }
    float ap[8];
    load8(a + kc, ap);
#pragma unroll
    for (int j = 0; j < 8; ++j) ap[j] = fmaxf(ap[j], 1e-8f);
#pragma unroll
    for (int al = 0; al < kMaxAlpha; ++al) {
      if (al < n_alpha) {
        float s[8], r1[8], r15[8];
        load8(s_table + (int64_t)al * K + kc, s);
        load8(rc + (int64_t)al * 2 * K + kc, r1);
        load8(rc + (int64_t)al * 2 * K + K + kc, r15);
        float smin = s[0], smax = s[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) {
          smin = fminf(smin, s[j]);
          smax = fmaxf(smax, s[j]);
        }
        const bool sok = smin >= 0x1p-14f && smax <= 0x1p14f;
        double sum = 0.0;
#pragma unroll
        for (int i = 0; i < kRB; ++i) {
          float X[8], D[8], v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) X[j] = x[i][j] * s[j];
          // from a finite (or infinite) amax the E8M0 byte is at most 253
          const uint32_t e8 = mx_e8m0_bits(quad_max_u(absmax8_bits(X)));
          const float sc = mx_scale_operand(e8);
          mx_unpack8_cvt(mx_pack8(X, sc), sc, D);
          if (sok && e8 - 16u <= 222u) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const uint32_t d = __float_as_uint(D[j]);
              const uint32_t m = (uint32_t)((int32_t)(d << 9) >> 31);   // all ones for c = 1.5 * 2^k
              const float r = __uint_as_float((__float_as_uint(r15[j]) & m) | (__float_as_uint(r1[j]) & ~m));
              v[j] = __uint_as_float(d & 0xFF800000u) * r;
            }
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = D[j] / s[j];
          }
          double q[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float t = (v[j] - x[i][j]) * ap[j];
            q[j] = (double)(t * t);
          }
          const double su = ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
          if (use[i]) sum += su;
        }
        acc[al] += sum;
      }
    }
  }
  __shared__ double red[kTasksPerBlock][kMaxAlpha];
#pragma unroll
  for (int al = 0; al < kMaxAlpha; ++al) {   // unrolled so acc stays in registers
    if (al < n_alpha) {
      double v = acc[al];
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
      if (lane == 0) red[wave][al] = v;
    }
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < n_alpha) part[(int64_t)t * gridDim.x + blockIdx.x] = (red[0][t] + red[1][t]) + (red[2][t] + red[3][t]);
}

// One wavefront per alpha sums that alpha's partials (a contiguous row of the [alpha,
// block] layout: lane-strided in block order, then wave_sum_f64), then thread 0 takes the
// first strict minimum.
__global__ __launch_bounds__(1024) void awq_finalize_kernel(const double* __restrict__ part, unsigned nblocks,
                                                            int n_alpha, double* __restrict__ err,
                                                            int32_t* __restrict__ best) {
  __shared__ double e[kMaxAlpha];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (wave < n_alpha) {
    const double* row = part + (int64_t)wave * nblocks;
    double acc = 0.0;
    // b = lane, lane + 64, ... in order; half batches (1024 threads leave 128 registers)
    for (unsigned b0 = lane; b0 < nblocks; b0 += 64 * (kLoadBatch / 2)) {
      double v[kLoadBatch / 2];
#pragma unroll
      for (int j = 0; j < kLoadBatch / 2; ++j) v[j] = row[min(b0 + 64 * j, nblocks - 1)];
#pragma unroll
      for (int j = 0; j < kLoadBatch / 2; ++j)
        if (b0 + 64 * j < nblocks) acc += v[j];
    }
    acc = wave_sum_f64(acc);
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

// ------------------------------------------------------------------ launch shape
struct AwqShape {
  int nchunk, ntasks;
  unsigned grid;
};
static AwqShape awq_shape(int64_t rows, int64_t K) {
  AwqShape sh;
  sh.nchunk = (int)((K + kTaskCols - 1) / kTaskCols);
  sh.ntasks = (int)((rows + kRB - 1) / kRB) * sh.nchunk;
  const unsigned g = (unsigned)((sh.ntasks + kTasksPerBlock - 1) / kTasksPerBlock);
  sh.grid = g < kSearchGridCap ? (g ? g : 1) : kSearchGridCap;
  return sh;
}

// Workspace: powers p [n_alpha, K] f64 | log sums [n_alpha, chunks] f64 |
// quotients [n_alpha, 2, K] f32 | search partials [n_alpha, grid] f64, each 16-byte aligned.
struct AwqLayout {
  size_t pw, logs, rc, part, total;
};
static size_t up16(size_t x) { return (x + 15) & ~(size_t)15; }
static AwqLayout awq_layout(int64_t rows, int64_t K, int n_alpha) {
  const size_t chunks = (size_t)((K + kChunk - 1) / kChunk);
  AwqLayout L;
  L.pw = 0;
  L.logs = up16(L.pw + (size_t)n_alpha * K * sizeof(double));
  L.rc = up16(L.logs + (size_t)n_alpha * chunks * sizeof(double));
  L.part = up16(L.rc + (size_t)n_alpha * 2 * K * sizeof(float));
  L.total = L.part + (size_t)awq_shape(rows, K).grid * n_alpha * sizeof(double);
  return L;
}

size_t awq_workspace_bytes(int64_t rows, int64_t K, int n_alpha) { return awq_layout(rows, K, n_alpha).total; }

void launch_awq(const void* W, int32_t w_dtype, int64_t rows, int64_t row_step, int64_t K, int64_t ldw,
                const float* a, const double* alphas, int n_alpha, float* s_table, double* err,
                int32_t* best, void* workspace, hipStream_t st) {
  const AwqLayout L = awq_layout(rows, K, n_alpha);
  char* ws = (char*)workspace;
  double* pw = (double*)(ws + L.pw);
  double* logs = (double*)(ws + L.logs);
  float* rc = (float*)(ws + L.rc);
  double* part = (double*)(ws + L.part);
  const dim3 tgrid((unsigned)((K + kChunk - 1) / kChunk), (unsigned)n_alpha);
  if (alphas) {
    Alphas al{};
    for (int i = 0; i < n_alpha; ++i) al.v[i] = alphas[i];
    hipLaunchKernelGGL(awq_pow_kernel, tgrid, dim3(kChunk), 0, st, a, (int)K, al, pw, logs);
    hipLaunchKernelGGL(awq_scale_kernel, tgrid, dim3(kChunk), 0, st, (const double*)pw, (const double*)logs,
                       (int)K, s_table, rc);
  } else {
    hipLaunchKernelGGL(awq_scale_kernel, tgrid, dim3(kChunk), 0, st, (const double*)nullptr,
                       (const double*)nullptr, (int)K, s_table, rc);
  }
  const AwqShape sh = awq_shape(rows, K);
  if (w_dtype == kBF16)
    hipLaunchKernelGGL(awq_search_kernel<uint16_t>, dim3(sh.grid), dim3(256), 0, st, (const uint16_t*)W, ldw,
                       row_step, (int)rows, (int)K, sh.nchunk, sh.ntasks, a, (const float*)s_table,
                       (const float*)rc, n_alpha, part);
  else
    hipLaunchKernelGGL(awq_search_kernel<float>, dim3(sh.grid), dim3(256), 0, st, (const float*)W, ldw, row_step,
                       (int)rows, (int)K, sh.nchunk, sh.ntasks, a, (const float*)s_table, (const float*)rc,
                       n_alpha, part);
  hipLaunchKernelGGL(awq_finalize_kernel, dim3(1), dim3(1024), 0, st, (const double*)part, sh.grid, n_alpha, err,
                     best);
}

}  // namespace gwb
