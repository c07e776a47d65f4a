// Reduction of the fused error kernels' per-block partial sums, and the streaming
// bandwidth ceilings the benchmark reports beside them.
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

// GWB_BLOCKS_PER_CU (1..64), when set, replaces every streaming kernel's own choice of
// resident blocks per compute unit (a measurement knob; unset in normal use).
static int blocks_per_cu_override() {
  static const int v = [] {
    const char* s = std::getenv("GWB_BLOCKS_PER_CU");
    int x = s ? std::atoi(s) : 0;
    return x > 0 && x <= 64 ? x : 0;
  }();
  return v;
}

unsigned stream_blocks(uint64_t units) { return stream_grid(units, 0); }

unsigned stream_grid(uint64_t units, int per_cu) {
  uint64_t need = (units + 255) / 256;
  if (need == 0) need = 1;
  const int bpc = blocks_per_cu_override() > 0 ? blocks_per_cu_override() : (per_cu > 0 ? per_cu : 8);
  const uint64_t cap = (uint64_t)compute_units_of_current_device() * (uint64_t)bpc;
  return (unsigned)(need < cap ? need : cap);
}

// part[2*i], part[2*i+1] for i < nblocks -> out[0] = sum w^2, out[1] = sum (w-d)^2,
// out[2] = 10 log10(out[0] / max(out[1], 1e-24)) (page export_gptq_cpu.py's
// 20 log10(||w|| / max(||w - deq||, 1e-12)), squared inside the log). One block of
// 1024 threads. The partials were just written by every XCD, so each load waits on the
// Infinity Cache: a thread issues kFinBatch independent loads per round (one round for
// up to 16384 partials) and sums them in index order, then each wavefront sums its lanes
// (wave_sum_f64) and thread 0 adds the 16 wavefront sums in order: deterministic for a
// given partial count.
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
  a = wave_sum_f64(a);
  b = wave_sum_f64(b);
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

// Streaming ceilings for the benchmark (not part of the method): eight 16-byte units per
// lane in flight, non-temporal loads of the large side, non-temporal 16-byte stores.
// Pattern: 0 copy (read `units` 16-byte units, write as many), 1 read only (one word per
// thread out), 2 quantize-shaped (read a 16-byte unit, write 4 bytes), 3 dequantize-shaped
// (read 4 bytes, write a 16-byte unit). STRIDED: grid-stride over the units; otherwise
// each block streams one contiguous range.
template <int PAT, bool STRIDED>
__global__ __launch_bounds__(256) void stream_bench_kernel(void* __restrict__ dst, const void* __restrict__ src,
                                                           uint64_t units) {
  constexpr int U = 8;
  uint64_t i, end, step;
  if constexpr (STRIDED) {
    i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    end = units;
    step = (uint64_t)gridDim.x * 256;
  } else {
    uint64_t per = (units + gridDim.x - 1) / gridDim.x;
    per = (per + 256 * U - 1) / (256 * U) * (256 * U);
    const uint64_t b0 = (uint64_t)blockIdx.x * per;
    i = b0 + threadIdx.x;
    end = b0 + per < units ? b0 + per : units;
    step = 256;
  }
  const U4* s16 = (const U4*)src;
  const uint32_t* s4 = (const uint32_t*)src;
  U4* d16 = (U4*)dst;
  uint32_t* d4 = (uint32_t*)dst;
  uint32_t acc = 0;
  for (; i + (U - 1) * step < end; i += U * step) {
    if constexpr (PAT == 3) {
      uint32_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = s4[i + u * step];
#pragma unroll
      for (int u = 0; u < U; ++u) st16_nt(d16 + i + u * step, U4{v[u], v[u] + 1, v[u] + 2, v[u] + 3});
    } else {
      U4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = ld16_nt(s16 + i + u * step);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if constexpr (PAT == 0) st16_nt(d16 + i + u * step, v[u]);
        else if constexpr (PAT == 1) acc ^= v[u].x ^ v[u].w;
        else d4[i + u * step] = v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
      }
    }
  }
  for (; i < end; i += step) {
    if constexpr (PAT == 3) {
      const uint32_t v = s4[i];
      st16_nt(d16 + i, U4{v, v + 1, v + 2, v + 3});
    } else {
      const U4 v = ld16_nt(s16 + i);
      if constexpr (PAT == 0) st16_nt(d16 + i, v);
      else if constexpr (PAT == 1) acc ^= v.x ^ v.w;
      else d4[i] = v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  if constexpr (PAT == 1) d4[(uint64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

template <bool STRIDED>
static void stream_bench_launch(int pattern, unsigned blocks, void* d, const void* s, uint64_t units, hipStream_t st) {
  if (pattern == 0) hipLaunchKernelGGL((stream_bench_kernel<0, STRIDED>), dim3(blocks), dim3(256), 0, st, d, s, units);
  else if (pattern == 1) hipLaunchKernelGGL((stream_bench_kernel<1, STRIDED>), dim3(blocks), dim3(256), 0, st, d, s, units);
  else if (pattern == 2) hipLaunchKernelGGL((stream_bench_kernel<2, STRIDED>), dim3(blocks), dim3(256), 0, st, d, s, units);
  else hipLaunchKernelGGL((stream_bench_kernel<3, STRIDED>), dim3(blocks), dim3(256), 0, st, d, s, units);
}

void launch_stream_bench(int pattern, bool strided, unsigned blocks, void* dst, const void* src, uint64_t units,
                         hipStream_t st) {
  if (strided) stream_bench_launch<true>(pattern, blocks, dst, src, units, st);
  else stream_bench_launch<false>(pattern, blocks, dst, src, units, st);
}

}  // namespace gwb
