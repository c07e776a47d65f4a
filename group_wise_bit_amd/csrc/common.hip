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
// 1024 threads. The partials were just written by every XCD, so each load waits on the
// Infinity Cache: a thread issues kFinBatch independent loads per round (one round for
// up to 16384 partials) and sums them in index order, then the wavefronts reduce by a
// fixed butterfly and wavefront 0 adds the 16 wavefront sums in order: deterministic for
// a given partial count.
constexpr int kFinThreads = 1024;
constexpr int kFinBatch = 16;
__global__ __launch_bounds__(kFinThreads) void err_finalize_kernel(const double2* __restrict__ part,
                                                                   unsigned nblocks, double* __restrict__ out) {
  __shared__ double sa[kFinThreads / 64], sb[kFinThreads / 64];
  double a = 0.0, b = 0.0;
  for (unsigned base = 0; base < nblocks; base += kFinBatch * kFinThreads) {
    double2 v[kFinBatch];
#pragma unroll
    for (int j = 0; j < kFinBatch; ++j) {
      const unsigned k = base + j * kFinThreads + threadIdx.x;
      v[j] = k < nblocks ? part[k] : double2{0.0, 0.0};
    }
#pragma unroll
    for (int j = 0; j < kFinBatch; ++j) {
      a += v[j].x;
      b += v[j].y;
    }
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) {
    a += __shfl_xor(a, m);
    b += __shfl_xor(b, m);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sa[w] = a;
    sb[w] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double w2 = 0.0, e2 = 0.0;
    for (int i = 0; i < kFinThreads / 64; ++i) {
      w2 += sa[i];
      e2 += sb[i];
    }
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
