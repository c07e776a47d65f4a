// 4-bit GPTQ quantize+pack, unpack+dequantize and fused reconstruction error.
// Page export_gptq_cpu.py: pack_int32, quantize_sym (vLLM uint4b8, w = (code-8)*scale,
// qzeros all 7) and quantize_asym (zp stored as itself).
//
// A block owns a tile of 64 weight rows (output channels n) x one group of G along K.
// Each lane takes 8 consecutive k of one row (one 128-bit bf16 load), so a row's
// group is G/8 lanes and its amax (or min/max) is a DPP reduction within a 16-lane
// row. The lane's 8 codes are one qweight word (r, n); words go through LDS so that
// the [K/8, N] int32 output is written as 256-byte runs along n.
//
// Codes need rint(fl(x / s)) with IEEE division. Per element the kernel forms
// q = x * y with y = fl(1/s) (one division per group): |q - x/s| <= |x/s| * 2^-22.9,
// and fl(x/s) is within |x/s| * 2^-24 of x/s, so when rint(q) is further than
// |q| * 2^-19 from a half-integer both round to the same integer. Otherwise (about one
// element in 10^4) the kernel divides exactly. |q| > 64 clamps either way.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gwb {

__device__ __forceinline__ float rint_div(float x, float s, float y) {
  float q = x * y;
  float n = rintf(q);
  float aq = fabsf(q);
  // fmaf only bounds a margin here; its rounding cannot make an unsafe case pass
  // because the margin (2^-19) is 8x the worst-case distance (2^-21.9).
  bool safe = aq > 64.0f || __builtin_fmaf(aq, 0x1p-19f, fabsf(q - n)) < 0.5f;
  if (!safe) n = rintf(x / s);
  return n;
}

template <int G>
struct Tile {
  static constexpr int L = G / 8;         // lanes per row-group
  static constexpr int RP = 256 / L;      // rows per pass
  static constexpr int P = 64 / RP;       // passes over the 64-row tile
  static constexpr int S = 68;            // LDS row stride of the [L][64] word tile
};

template <bool SYM, int G, typename TIn>
__global__ __launch_bounds__(256) void gptq_quant_kernel(const TIn* __restrict__ W, int64_t ldw,
                                                         int N, int ntiles_n, int ngroups,
                                                         uint32_t* __restrict__ qweight,
                                                         _Float16* __restrict__ scales,
                                                         uint32_t* __restrict__ qzeros,
                                                         int32_t* __restrict__ g_idx) {
  using T = Tile<G>;
  __shared__ uint32_t qtile[T::L * T::S];
  __shared__ float stile[64];
  __shared__ uint8_t ztile[64];
  const int t = threadIdx.x;
  const int nt = blockIdx.x / ngroups;
  const int g = blockIdx.x - nt * ngroups;
  const int unit = t % T::L;
#pragma unroll
  for (int p = 0; p < T::P; ++p) {
    const int rl = p * T::RP + t / T::L;
    const int n = nt * 64 + rl;
    if (n < N) {
      float x[8];
      load8(W + (int64_t)n * ldw + (int64_t)g * G + unit * 8, x);
      float s, y, zp;
      if constexpr (SYM) {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
        amax = lanes_max<T::L>(amax);
        s = fmaxf(amax / 8.0f, 1e-9f);
        zp = 8.0f;
      } else {
        float mx = x[0], mn = x[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) { mx = fmaxf(mx, x[i]); mn = fminf(mn, x[i]); }
        mx = lanes_max<T::L>(mx);
        mn = lanes_min<T::L>(mn);
        s = fmaxf(mx - mn, 1e-9f) / 15.0f;
        zp = fminf(fmaxf(rintf(-mn / s), 0.0f), 15.0f);
      }
      y = 1.0f / s;
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float c = fminf(fmaxf(rint_div(x[i], s, y) + zp, 0.0f), 15.0f);
        word |= (uint32_t)c << (4 * i);
      }
      qtile[unit * T::S + rl] = word;
      if (unit == 0) {
        stile[rl] = s;
        ztile[rl] = (uint8_t)zp;
      }
    }
  }
  __syncthreads();
  const int n0 = nt * 64;
  {  // qweight rows 16g.. of [K/8, N]: L rows x 64 words, 16 threads x 16 bytes per row
    const int r = t / 16, c4 = (t % 16) * 4;
    if (r < T::L && n0 + c4 < N) {
      const uint32_t* src = &qtile[r * T::S + c4];
      U4 v{src[0], src[1], src[2], src[3]};
      st16(qweight + (int64_t)(g * T::L + r) * N + n0 + c4, v);
    }
  }
  if (t < 64 && n0 + t < N) scales[(int64_t)g * N + n0 + t] = (_Float16)stile[t];
  if (t < 8 && n0 + 8 * t < N) {
    uint32_t w = 0x77777777u;
    if constexpr (!SYM) {
      w = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) w |= (uint32_t)ztile[8 * t + i] << (4 * i);
    }
    qzeros[(int64_t)g * (N / 8) + nt * 8 + t] = w;
  }
  if (g_idx && nt == 0 && t < G) g_idx[g * G + t] = g;
}

// Unpack + dequantize, grid-stride over tiles. SINK as in mxfp4.hip.
template <int SINK, bool SYM, int G, typename TOut, typename TW>
__global__ __launch_bounds__(256) void gptq_dequant_kernel(const uint32_t* __restrict__ qweight,
                                                           const _Float16* __restrict__ scales,
                                                           const uint32_t* __restrict__ qzeros,
                                                           int N, int ntiles_n, int ngroups,
                                                           TOut* __restrict__ out, int64_t ldo,
                                                           const TW* __restrict__ W, int64_t ldw,
                                                           double* __restrict__ part) {
  using T = Tile<G>;
  __shared__ uint32_t qtile[T::L * T::S];
  __shared__ float stile[64];
  __shared__ uint32_t ztile[8];
  const int t = threadIdx.x;
  const int unit = t % T::L;
  double sw = 0.0, se = 0.0;
  const int ntiles = ntiles_n * ngroups;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int nt = tile / ngroups;
    const int g = tile - nt * ngroups;
    const int n0 = nt * 64;
    {
      const int r = t / 16, c4 = (t % 16) * 4;
      if (r < T::L && n0 + c4 < N) {
        U4 v = ld16(qweight + (int64_t)(g * T::L + r) * N + n0 + c4);
        uint32_t* dst = &qtile[r * T::S + c4];
        dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
      }
    }
    if (t < 64 && n0 + t < N) stile[t] = (float)scales[(int64_t)g * N + n0 + t];
    if (!SYM && t < 8 && n0 + 8 * t < N) ztile[t] = qzeros[(int64_t)g * (N / 8) + nt * 8 + t];
    __syncthreads();
#pragma unroll
    for (int p = 0; p < T::P; ++p) {
      const int rl = p * T::RP + t / T::L;
      const int n = n0 + rl;
      if (n < N) {
        const uint32_t word = qtile[unit * T::S + rl];
        const float s = stile[rl];
        float z = 8.0f;
        if constexpr (!SYM) z = (float)((ztile[rl / 8] >> (4 * (rl % 8))) & 0xFu);
        float d[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) d[i] = ((float)((word >> (4 * i)) & 0xFu) - z) * s;
        const int64_t k0 = (int64_t)g * G + unit * 8;
        if constexpr (SINK == kStore) {
          store8(out + (int64_t)n * ldo + k0, d);
        } else {
          float x[8];
          load8(W + (int64_t)n * ldw + k0, x);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            double xd = (double)x[i];
            double ed = (double)(x[i] - d[i]);
            sw = fma(xd, xd, sw);
            se = fma(ed, ed, se);
          }
        }
      }
    }
    __syncthreads();
  }
  if constexpr (SINK == kErr) block_sum2_store<256>(sw, se, part);
}

// ------------------------------------------------------------------ launchers
template <bool SYM, int G>
static void quant_g(const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw, void* qw,
                    void* sc, void* qz, void* gi, hipStream_t st) {
  int ntn = (int)((N + 63) / 64), ng = (int)(K / G);
  dim3 grid((unsigned)(ntn * ng));
  if (w_dtype == kBF16)
    hipLaunchKernelGGL((gptq_quant_kernel<SYM, G, uint16_t>), grid, dim3(256), 0, st, (const uint16_t*)W,
                       ldw, (int)N, ntn, ng, (uint32_t*)qw, (_Float16*)sc, (uint32_t*)qz, (int32_t*)gi);
  else
    hipLaunchKernelGGL((gptq_quant_kernel<SYM, G, float>), grid, dim3(256), 0, st, (const float*)W, ldw,
                       (int)N, ntn, ng, (uint32_t*)qw, (_Float16*)sc, (uint32_t*)qz, (int32_t*)gi);
}

template <bool SYM>
static void quant_s(int group, const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw,
                    void* qw, void* sc, void* qz, void* gi, hipStream_t st) {
  if (group == 32) quant_g<SYM, 32>(W, w_dtype, N, K, ldw, qw, sc, qz, gi, st);
  else if (group == 64) quant_g<SYM, 64>(W, w_dtype, N, K, ldw, qw, sc, qz, gi, st);
  else quant_g<SYM, 128>(W, w_dtype, N, K, ldw, qw, sc, qz, gi, st);
}

void launch_gptq_quant(bool sym, int group, const void* W, int32_t w_dtype, int64_t N, int64_t K,
                       int64_t ldw, void* qweight, void* scales, void* qzeros, void* g_idx,
                       hipStream_t st) {
  if (sym) quant_s<true>(group, W, w_dtype, N, K, ldw, qweight, scales, qzeros, g_idx, st);
  else quant_s<false>(group, W, w_dtype, N, K, ldw, qweight, scales, qzeros, g_idx, st);
}

static unsigned tiles_of(int group, int64_t N, int64_t K) {
  return (unsigned)(((N + 63) / 64) * (K / group));
}

template <int SINK, bool SYM, int G, typename TOut, typename TW>
static void deq_launch(unsigned grid, const void* qw, const void* sc, const void* qz, int64_t N, int64_t K,
                       void* out, int64_t ldo, const void* W, int64_t ldw, double* part, hipStream_t st) {
  int ntn = (int)((N + 63) / 64), ng = (int)(K / G);
  hipLaunchKernelGGL((gptq_dequant_kernel<SINK, SYM, G, TOut, TW>), dim3(grid), dim3(256), 0, st,
                     (const uint32_t*)qw, (const _Float16*)sc, (const uint32_t*)qz, (int)N, ntn, ng,
                     (TOut*)out, ldo, (const TW*)W, ldw, part);
}

template <int SINK, bool SYM, typename TOut, typename TW>
static void deq_g(int group, unsigned grid, const void* qw, const void* sc, const void* qz, int64_t N,
                  int64_t K, void* out, int64_t ldo, const void* W, int64_t ldw, double* part,
                  hipStream_t st) {
  if (group == 32) deq_launch<SINK, SYM, 32, TOut, TW>(grid, qw, sc, qz, N, K, out, ldo, W, ldw, part, st);
  else if (group == 64) deq_launch<SINK, SYM, 64, TOut, TW>(grid, qw, sc, qz, N, K, out, ldo, W, ldw, part, st);
  else deq_launch<SINK, SYM, 128, TOut, TW>(grid, qw, sc, qz, N, K, out, ldo, W, ldw, part, st);
}

void launch_gptq_dequant(bool sym, int group, const void* qweight, const void* scales,
                         const void* qzeros, int64_t N, int64_t K, void* out, int32_t out_dtype,
                         int64_t ldo, hipStream_t st) {
  unsigned grid = tiles_of(group, N, K);
  if (sym) {
    if (out_dtype == kBF16)
      deq_g<kStore, true, uint16_t, uint16_t>(group, grid, qweight, scales, qzeros, N, K, out, ldo, nullptr, 0, nullptr, st);
    else
      deq_g<kStore, true, float, uint16_t>(group, grid, qweight, scales, qzeros, N, K, out, ldo, nullptr, 0, nullptr, st);
  } else {
    if (out_dtype == kBF16)
      deq_g<kStore, false, uint16_t, uint16_t>(group, grid, qweight, scales, qzeros, N, K, out, ldo, nullptr, 0, nullptr, st);
    else
      deq_g<kStore, false, float, uint16_t>(group, grid, qweight, scales, qzeros, N, K, out, ldo, nullptr, 0, nullptr, st);
  }
}

unsigned gptq_err_blocks(int group, int64_t N, int64_t K) {
  unsigned t = tiles_of(group, N, K);
  return t < kErrGridCap ? (t ? t : 1) : kErrGridCap;   // tiles, capped: fixed by the shape
}

void launch_gptq_err(bool sym, int group, const void* W, int32_t w_dtype, int64_t N, int64_t K,
                     int64_t ldw, const void* qweight, const void* scales, const void* qzeros,
                     double* part, hipStream_t st) {
  unsigned grid = gptq_err_blocks(group, N, K);
  if (sym) {
    if (w_dtype == kBF16)
      deq_g<kErr, true, float, uint16_t>(group, grid, qweight, scales, qzeros, N, K, nullptr, 0, W, ldw, part, st);
    else
      deq_g<kErr, true, float, float>(group, grid, qweight, scales, qzeros, N, K, nullptr, 0, W, ldw, part, st);
  } else {
    if (w_dtype == kBF16)
      deq_g<kErr, false, float, uint16_t>(group, grid, qweight, scales, qzeros, N, K, nullptr, 0, W, ldw, part, st);
    else
      deq_g<kErr, false, float, float>(group, grid, qweight, scales, qzeros, N, K, nullptr, 0, W, ldw, part, st);
  }
}

}  // namespace gwb
