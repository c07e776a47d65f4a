// Reduction of the fused error kernels' per-block partial sums, and the bandwidth
// reference copy used by the benchmark.
#include <atomic>
#include <cstdlib>

#include "device_common.hpp"
#include "kernels.hpp"

namespace gwb {

static int compute_units_of_current_device() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

static int blocks_per_cu() {
  static const int v = [] {
    const char* s = std::getenv("GWB_BLOCKS_PER_CU");
    int x = s ? std::atoi(s) : 0;
    return x > 0 && x <= 64 ? x : 8;
  }();
  return v;
}

unsigned stream_blocks(uint64_t units) {
  uint64_t need = (units + 255) / 256;
  if (need == 0) need = 1;
  const uint64_t cap = (uint64_t)compute_units_of_current_device() * (uint64_t)blocks_per_cu();
  return (unsigned)(need < cap ? need : cap);
}

// part[2*i], part[2*i+1] for i < nblocks -> out[0] = sum w^2, out[1] = sum (w-d)^2,
// out[2] = 10 log10(out[0] / max(out[1], 1e-24)) (page export_gptq_cpu.py's
// 20 log10(||w|| / max(||w - deq||, 1e-12)), squared inside the log). One block of
// 1024 threads; each thread sums a fixed strided subset with four independent chains,
// then a fixed tree: deterministic for a given partial count.
constexpr int kFinThreads = 1024;
__global__ __launch_bounds__(kFinThreads) void err_finalize_kernel(const double2* __restrict__ part,
                                                                   unsigned nblocks, double* __restrict__ out) {
  __shared__ double sa[kFinThreads], sb[kFinThreads];
  double a[4] = {0.0, 0.0, 0.0, 0.0}, b[4] = {0.0, 0.0, 0.0, 0.0};
  unsigned i = threadIdx.x;
  for (; i + 3 * kFinThreads < nblocks; i += 4 * kFinThreads) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double2 v = part[i + j * kFinThreads];
      a[j] += v.x;
      b[j] += v.y;
    }
  }
  for (; i < nblocks; i += kFinThreads) {
    const double2 v = part[i];
    a[0] += v.x;
    b[0] += v.y;
  }
  sa[threadIdx.x] = (a[0] + a[1]) + (a[2] + a[3]);
  sb[threadIdx.x] = (b[0] + b[1]) + (b[2] + b[3]);
  __syncthreads();
  for (int s = kFinThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      sa[threadIdx.x] += sa[threadIdx.x + s];
      sb[threadIdx.x] += sb[threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double w2 = sa[0], e2 = sb[0];
    out[0] = w2;
    out[1] = e2;
    out[2] = w2 == 0.0 ? -__builtin_inf() : 10.0 * log10(w2 / fmax(e2, 1e-24));
  }
}

void launch_err_finalize(const double* part, unsigned nblocks, double* out, hipStream_t st) {
  hipLaunchKernelGGL(err_finalize_kernel, dim3(1), dim3(kFinThreads), 0, st, (const double2*)part, nblocks, out);
}

__global__ __launch_bounds__(256) void stream_copy_kernel(U4* __restrict__ dst, const U4* __restrict__ src,
                                                          uint64_t n16) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

void launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t st) {
  uint64_t n16 = bytes / 16;
  uint64_t g = (n16 + 255) / 256;
  unsigned grid = (unsigned)(g < kStreamGridCap ? (g ? g : 1) : kStreamGridCap);
  hipLaunchKernelGGL(stream_copy_kernel, dim3(grid), dim3(256), 0, st, (U4*)dst, (const U4*)src, n16);
}

}  // namespace gwb
