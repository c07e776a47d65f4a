// 4-bit GPTQ quantize+pack, unpack+dequantize and fused reconstruction error.
// Page export_gptq_cpu.py: pack_int32, quantize_sym (vLLM uint4b8, w = (code-8)*scale,
// qzeros all 7) and quantize_asym (zp stored as itself).
//
// A tile is 32 weight rows (output channels n) x 512 along K. Each lane takes 8
// consecutive k of one row (one 128-bit bf16 load), so a group of G is G/8 adjacent
// lanes and its amax (or min/max) is a DPP reduction within a 16-lane row, while each
// load instruction of a wavefront reads 1 KB of one row (long DRAM runs). A lane's 8
// codes are one qweight word (r, n); words go through LDS so that the [K/8, N] int32
// output leaves as 128-byte runs along n.
//
// Codes need rint(fl(x / s)) with IEEE division. Per element the kernel forms
// q = x * y with y the hardware reciprocal of s (within 1 ulp of 1/s), so
// |q - x/s| <= |x/s| * 1.5 * 2^-23, and fl(x/s) is within |x/s| * 2^-24 of x/s: when
// rint(q) is further than |q| * 2^-19 from a half-integer, both round to the same
// integer. Otherwise (about one element in 10^4) the kernel divides exactly. |q| > 64
// clamps either way.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gwb {

typedef short s16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short gq_u16x2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------- group reductions
// amax of 8 weights as float32 bits (|x| orders like its bits).
__device__ __forceinline__ uint32_t gq_absmax_bits(const Raw8<uint16_t>& r) {
  const uint32_t m = 0x7FFF7FFFu;
  gq_u16x2_t a = __builtin_bit_cast(gq_u16x2_t, r.v.x & m), b = __builtin_bit_cast(gq_u16x2_t, r.v.y & m);
  gq_u16x2_t c = __builtin_bit_cast(gq_u16x2_t, r.v.z & m), d = __builtin_bit_cast(gq_u16x2_t, r.v.w & m);
  gq_u16x2_t e = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  const uint32_t lo = e[0], hi = e[1];
  return (lo > hi ? lo : hi) << 16;
}
__device__ __forceinline__ uint32_t gq_absmax_bits(const Raw8<float>& r) {
  const uint32_t m = 0x7FFFFFFFu;
  uint32_t a = max(max(r.a.x & m, r.a.y & m), max(r.a.z & m, r.a.w & m));
  uint32_t b = max(max(r.b.x & m, r.b.y & m), max(r.b.z & m, r.b.w & m));
  return max(a, b);
}
template <int LANES>
__device__ __forceinline__ uint32_t lanes_max_u(uint32_t x) {
  if constexpr (LANES >= 2) x = max(x, dpp_read_u<kDppXor1>(x));
  if constexpr (LANES >= 4) x = max(x, dpp_read_u<kDppXor2>(x));
  if constexpr (LANES >= 8) x = max(x, dpp_read_u<kDppHalfMirror>(x));
  if constexpr (LANES >= 16) x = max(x, dpp_read_u<kDppMirror>(x));
  return x;
}
template <int LANES>
__device__ __forceinline__ int lanes_min_i(int x) {
  if constexpr (LANES >= 2) x = min(x, (int)dpp_read_u<kDppXor1>((uint32_t)x));
  if constexpr (LANES >= 4) x = min(x, (int)dpp_read_u<kDppXor2>((uint32_t)x));
  if constexpr (LANES >= 8) x = min(x, (int)dpp_read_u<kDppHalfMirror>((uint32_t)x));
  if constexpr (LANES >= 16) x = min(x, (int)dpp_read_u<kDppMirror>((uint32_t)x));
  return x;
}
template <int LANES>
__device__ __forceinline__ int lanes_max_i(int x) {
  if constexpr (LANES >= 2) x = max(x, (int)dpp_read_u<kDppXor1>((uint32_t)x));
  if constexpr (LANES >= 4) x = max(x, (int)dpp_read_u<kDppXor2>((uint32_t)x));
  if constexpr (LANES >= 8) x = max(x, (int)dpp_read_u<kDppHalfMirror>((uint32_t)x));
  if constexpr (LANES >= 16) x = max(x, (int)dpp_read_u<kDppMirror>((uint32_t)x));
  return x;
}

// Signed-order keys: key(h) = h ^ ((h >> 15) & 0x7FFF) as int16 orders bf16 bit
// patterns h like their values (-0 just below +0); the map is its own inverse.
__device__ __forceinline__ s16x2_t bf16_keys(uint32_t w) {
  const s16x2_t h = __builtin_bit_cast(s16x2_t, w);
  return h ^ ((h >> (short)15) & (short)0x7FFF);
}
__device__ __forceinline__ float key_to_f32(int k) {
  const int h = k ^ ((k >> 15) & 0x7FFF);
  return __uint_as_float((uint32_t)h << 16);
}
template <int LANES>
__device__ __forceinline__ void gq_minmax(const Raw8<uint16_t>& r, float& mn, float& mx) {
  const s16x2_t a = bf16_keys(r.v.x), b = bf16_keys(r.v.y), c = bf16_keys(r.v.z), d = bf16_keys(r.v.w);
  const s16x2_t lo = __builtin_elementwise_min(__builtin_elementwise_min(a, b), __builtin_elementwise_min(c, d));
  const s16x2_t hi = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  const int kmin = lanes_min_i<LANES>(min((int)lo[0], (int)lo[1]));
  const int kmax = lanes_max_i<LANES>(max((int)hi[0], (int)hi[1]));
  mn = key_to_f32(kmin);
  mx = key_to_f32(kmax);
}
template <int LANES>
__device__ __forceinline__ void gq_minmax(const Raw8<float>& r, float& mn, float& mx) {
  float x[8];
  to_f32(r, x);
  mn = x[0];
  mx = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
  mn = lanes_min<LANES>(mn);
  mx = lanes_max<LANES>(mx);
}

// ------------------------------------------------------------- codes
// 8 codes clamp(rint(fl(x / s)) + zp, 0, 15) packed into one word (code i in bits 4i..).
// A |q| so large that the margin test fails (only in degenerate groups) takes the exact
// path too.
__device__ __forceinline__ uint32_t gq_word(const float* x, float s, float zp) {
  const float y = __builtin_amdgcn_rcpf(s);
  float n[8];
  bool ok = true;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q = x[i] * y;
    n[i] = rintf(q);
    // fmaf only bounds a margin: its rounding cannot pass an unsafe case, the margin
    // being 8x the worst-case distance
    ok &= __builtin_fmaf(fabsf(q), 0x1p-19f, fabsf(q - n[i])) < 0.5f;
  }
  if (!ok) {
#pragma unroll
    for (int i = 0; i < 8; ++i) n[i] = rintf(x[i] / s);
  }
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= (uint32_t)__builtin_amdgcn_fmed3f(n[i] + zp, 0.0f, 15.0f) << (4 * i);
  return w;
}

// Tile: 32 rows x 512 k. Wave w holds rows 8w..8w+7; lane l holds k = k0 + 8l..8l+7 of
// each, so every load instruction of a wave reads 1 KB of one row and a 128-wide group
// is 16 adjacent lanes. qweight words meet in LDS as [64 r][32 n] and leave as 128-byte
// runs along n.
constexpr int kTN = 32, kTK = 512, kTR = kTK / 8;
constexpr int kQS = kTN + 1;                        // LDS row stride (words) of [kTR][kTN]

template <int G>
struct TileG {
  static constexpr int L = G / 8;                   // lanes per group
  static constexpr int NG = kTK / G;                // groups per tile row
};

template <bool SYM, int G, typename TIn>
__global__ __launch_bounds__(256) void gptq_quant_kernel(const TIn* __restrict__ W, int64_t ldw,
                                                         int N, int K, int ntk,
                                                         uint32_t* __restrict__ qweight,
                                                         _Float16* __restrict__ scales,
                                                         uint32_t* __restrict__ qzeros,
                                                         int32_t* __restrict__ g_idx) {
  using T = TileG<G>;
  __shared__ uint32_t qtile[kTR * kQS];
  __shared__ float stile[T::NG * kTN];
  __shared__ uint8_t ztile[T::NG * kTN];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int nt = blockIdx.x / ntk, kt = blockIdx.x - nt * ntk;
  const int n0 = nt * kTN, k0 = kt * kTK;
  const int k = k0 + lane * 8;
  const bool kok = k < K;                           // whole groups: K % G == 0
  Raw8<TIn> raw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int n = n0 + wave * 8 + i;
    if (kok && n < N) raw[i] = load_raw8(W + (int64_t)n * ldw + k);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rl = wave * 8 + i;
    if (kok && n0 + rl < N) {
      float x[8];
      to_f32(raw[i], x);
      float s, zp;
      if constexpr (SYM) {
        const float amax = __uint_as_float(lanes_max_u<T::L>(gq_absmax_bits(raw[i])));
        s = fmaxf(amax * 0.125f, 1e-9f);            // amax / 8: exact scaling by 2^-3
        zp = 8.0f;
      } else {
        float mn, mx;
        gq_minmax<T::L>(raw[i], mn, mx);
        s = fmaxf(mx - mn, 1e-9f) / 15.0f;
        zp = __builtin_amdgcn_fmed3f(rintf(-mn / s), 0.0f, 15.0f);
      }
      qtile[lane * kQS + rl] = gq_word(x, s, zp);
      if ((lane % T::L) == 0) {
        stile[(lane / T::L) * kTN + rl] = s;
        ztile[(lane / T::L) * kTN + rl] = (uint8_t)zp;
      }
    }
  }
  __syncthreads();
  {  // qweight [K/8, N]: 64 r-rows x 32 words, 8 words (32 bytes) per thread
    const int r = t >> 2, c8 = (t & 3) * 8;
    if (k0 / 8 + r < K / 8 && n0 + c8 < N) {
      const uint32_t* src = &qtile[r * kQS + c8];
      uint32_t* dst = qweight + (int64_t)(k0 / 8 + r) * N + n0 + c8;
      st16(dst, U4{src[0], src[1], src[2], src[3]});
      st16(dst + 4, U4{src[4], src[5], src[6], src[7]});
    }
  }
  for (int e = t; e < T::NG * kTN; e += 256) {   // scales [K/G, N]
    const int gl = e / kTN, rl = e % kTN;
    if (k0 + gl * G < K && n0 + rl < N) scales[(int64_t)(k0 / G + gl) * N + n0 + rl] = (_Float16)stile[e];
  }
  static_assert(T::NG * (kTN / 8) <= 256, "one qzeros word per thread");
  if (t < T::NG * (kTN / 8)) {   // qzeros [K/G, N/8]
    const int gl = t / (kTN / 8), q = t % (kTN / 8);
    if (k0 + gl * G < K && n0 + 8 * q < N) {
      uint32_t w = 0x77777777u;
      if constexpr (!SYM) {
        w = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) w |= (uint32_t)ztile[gl * kTN + 8 * q + i] << (4 * i);
      }
      qzeros[(int64_t)(k0 / G + gl) * (N / 8) + n0 / 8 + q] = w;
    }
  }
  if (g_idx && nt == 0) {
    for (int kk = t; kk < kTK; kk += 256)
      if (k0 + kk < K) g_idx[k0 + kk] = (k0 + kk) / G;
  }
}

// ------------------------------------------------------------- dequantize
// Same tile. The 64 x 32 qweight words come in as 128-byte runs through LDS; each lane
// then dequantizes 8 rows x 8 k and a wave writes 1 KB of one row per store. Blocks
// walk tiles grid-stride (SINK == kErr keeps its partial count fixed by the shape).
template <int SINK, bool SYM, int G, typename TOut, typename TW>
__global__ __launch_bounds__(256) void gptq_dequant_kernel(const uint32_t* __restrict__ qweight,
                                                           const _Float16* __restrict__ scales,
                                                           const uint32_t* __restrict__ qzeros,
                                                           int N, int K, int ntk, int ntiles,
                                                           TOut* __restrict__ out, int64_t ldo,
                                                           const TW* __restrict__ W, int64_t ldw,
                                                           double* __restrict__ part) {
  using T = TileG<G>;
  __shared__ uint32_t qtile[kTR * kQS];
  __shared__ float stile[T::NG * kTN];
  __shared__ uint32_t ztile[T::NG * (kTN / 8)];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  double sw = 0.0, se = 0.0;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int nt = tile / ntk, kt = tile - nt * ntk;
    const int n0 = nt * kTN, k0 = kt * kTK;
    {
      const int r = t >> 2, c8 = (t & 3) * 8;
      if (k0 / 8 + r < K / 8 && n0 + c8 < N) {
        const uint32_t* src = qweight + (int64_t)(k0 / 8 + r) * N + n0 + c8;
        const U4 a = ld16_nt(src), b = ld16_nt(src + 4);
        uint32_t* dst = &qtile[r * kQS + c8];
        dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
        dst[4] = b.x; dst[5] = b.y; dst[6] = b.z; dst[7] = b.w;
      }
    }
    for (int e = t; e < T::NG * kTN; e += 256) {
      const int gl = e / kTN, rl = e % kTN;
      if (k0 + gl * G < K && n0 + rl < N) stile[e] = (float)scales[(int64_t)(k0 / G + gl) * N + n0 + rl];
    }
    if (!SYM && t < T::NG * (kTN / 8)) {
      const int gl = t / (kTN / 8), q = t % (kTN / 8);
      if (k0 + gl * G < K && n0 + 8 * q < N) ztile[t] = qzeros[(int64_t)(k0 / G + gl) * (N / 8) + n0 / 8 + q];
    }
    __syncthreads();
    const int k = k0 + lane * 8;
    if (k < K) {
      const int gl = lane / T::L;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rl = wave * 8 + i;
        const int n = n0 + rl;
        if (n < N) {
          const uint32_t word = qtile[lane * kQS + rl];
          const float s = stile[gl * kTN + rl];
          float z = 8.0f;
          if constexpr (!SYM) z = (float)((ztile[gl * (kTN / 8) + rl / 8] >> (4 * (rl % 8))) & 0xFu);
          const uint32_t ev = word & 0x0F0F0F0Fu, od = (word >> 4) & 0x0F0F0F0Fu;
          // byte-to-float conversions (v_cvt_f32_ubyte0..3)
          const float c[8] = {(float)(ev & 0xFFu), (float)(od & 0xFFu), (float)((ev >> 8) & 0xFFu),
                              (float)((od >> 8) & 0xFFu), (float)((ev >> 16) & 0xFFu), (float)((od >> 16) & 0xFFu),
                              (float)(ev >> 24), (float)(od >> 24)};
          float d[8];
          if (__builtin_isfinite(s) && s != 0.0f) {
            // (c - z) * s is exact in float32, so c*s - z*s as one fma rounds it exactly
            const float nzs = -(z * s);
#pragma unroll
            for (int j = 0; j < 8; ++j) d[j] = __builtin_fmaf(c[j], s, nzs);
          } else {
            // fp16 scale overflowed or underflowed: the page's (c - z) * s gives +-inf
            // (NaN at c == z), or a zero carrying the sign of c - z
#pragma unroll
            for (int j = 0; j < 8; ++j) d[j] = (c[j] - z) * s;
          }
          if constexpr (SINK == kStore) {
            store8(out + (int64_t)n * ldo + k, d);
          } else {
            float x[8];
            to_f32(load_raw8(W + (int64_t)n * ldw + k), x);
            acc_err8(x, d, sw, se);
          }
        }
      }
    }
    __syncthreads();
  }
  if constexpr (SINK == kErr) block_sum2_store<256>(sw, se, part);
}

// ------------------------------------------------------------------ launchers
static int ntk_of(int64_t K) { return (int)((K + kTK - 1) / kTK); }
static unsigned tiles_of(int64_t N, int64_t K) { return (unsigned)(((N + kTN - 1) / kTN) * ntk_of(K)); }

template <bool SYM, int G>
static void quant_g(const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw, void* qw,
                    void* sc, void* qz, void* gi, hipStream_t st) {
  const dim3 grid(tiles_of(N, K));
  if (w_dtype == kBF16)
    hipLaunchKernelGGL((gptq_quant_kernel<SYM, G, uint16_t>), grid, dim3(256), 0, st, (const uint16_t*)W,
                       ldw, (int)N, (int)K, ntk_of(K), (uint32_t*)qw, (_Float16*)sc, (uint32_t*)qz, (int32_t*)gi);
  else
    hipLaunchKernelGGL((gptq_quant_kernel<SYM, G, float>), grid, dim3(256), 0, st, (const float*)W, ldw,
                       (int)N, (int)K, ntk_of(K), (uint32_t*)qw, (_Float16*)sc, (uint32_t*)qz, (int32_t*)gi);
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

template <int SINK, bool SYM, int G, typename TOut, typename TW>
static void deq_launch(unsigned grid, const void* qw, const void* sc, const void* qz, int64_t N, int64_t K,
                       void* out, int64_t ldo, const void* W, int64_t ldw, double* part, hipStream_t st) {
  hipLaunchKernelGGL((gptq_dequant_kernel<SINK, SYM, G, TOut, TW>), dim3(grid), dim3(256), 0, st,
                     (const uint32_t*)qw, (const _Float16*)sc, (const uint32_t*)qz, (int)N, (int)K, ntk_of(K),
                     (int)tiles_of(N, K), (TOut*)out, ldo, (const TW*)W, ldw, part);
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
  const unsigned grid = tiles_of(N, K);
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

// One block per tile (the error partials follow the tiles), capped for very large
// matrices: fixed by the shape alone.
unsigned gptq_err_blocks(int group, int64_t N, int64_t K) {
  (void)group;
  const unsigned t = tiles_of(N, K);
  const unsigned cap = 16 * kErrGridCap;
  return t < cap ? (t ? t : 1) : cap;
}

void launch_gptq_err(bool sym, int group, const void* W, int32_t w_dtype, int64_t N, int64_t K,
                     int64_t ldw, const void* qweight, const void* scales, const void* qzeros,
                     double* part, hipStream_t st) {
  const unsigned grid = gptq_err_blocks(group, N, K);
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
