// GPTQ with act-order groups (desc_act): the groups are formed over the input channels
// taken in a caller-given order, qweight stays in channel order and g_idx[k] names the
// group of channel k. Page export_gptq_cpu.py stores g_idx and writes desc_act into the
// checkpoint config; its per-group formulas (quantize_sym / quantize_asym) are used
// unchanged on those groups, and a consumer reads channel k with the scale and zero
// point of group g_idx[k].
//
// Quantization: (1) g_idx[perm[j]] = j / G; (2) per row, the weight row in LDS and each
// group reduced over its channels perm[gG .. gG + G - 1], giving the float32 scale and
// zero point of every (row, group) in a workspace; (3) the codes in channel order, in the
// tile layout of gptq.hip (32 rows x 512 k, qweight words transposed through LDS), each
// channel with the parameters of its group; the codes are those of the IEEE quotient
// x / s the page divides, found through the reciprocal with exact division near
// rounding boundaries.
// Dequantization and the fused error use the same tile with each channel's group read
// from g_idx. Both tile kernels keep every group of their 32-row band in LDS, so K / G is
// limited to kActMaxGroups; quantization also holds one weight row in LDS (64 KB).
//
// perm must be a permutation of 0..K-1 and g_idx values must lie in [0, K/G): other
// values are clamped into range (no access leaves its buffer) and give unspecified codes.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gwb {

namespace {
constexpr int kTN = 32, kTK = 512, kTR = kTK / 8;   // the gptq.hip tile
constexpr int kQS = kTN + 1;
// Per-group tables in LDS are [group][kPS]: lanes of one lookup share the row and differ
// in the group, so a stride of 33 words spreads them over the banks (32 would put every
// lane on one bank).
constexpr int kPS = kTN + 1;

__device__ __forceinline__ uint32_t clamp_idx(int32_t v, uint32_t n) {
  return v < 0 ? 0u : ((uint32_t)v >= n ? n - 1 : (uint32_t)v);
}
// Staging loops issue their loads in batches of kBatch before storing any of them, so a
// thread waits for one memory round trip per batch rather than one per element.
constexpr int kBatch = 8;
template <int NT = 256>
__device__ __forceinline__ void stage16(U4* __restrict__ dst, const U4* __restrict__ src, int n) {
  for (int c0 = threadIdx.x; c0 < n; c0 += NT * kBatch) {
    U4 v[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      if (c0 + NT * q < n) v[q] = ld16(src + c0 + NT * q);
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      if (c0 + NT * q < n) dst[c0 + NT * q] = v[q];
  }
}
// Threads of a parameters block: one weight row each, so 128 threads let a CU hold 16
// rows in LDS (160 KB at 10 KB a row) and keep more of them loading while others reduce.
constexpr int kParamThreads = 128;
}  // namespace

// g_idx[perm[j]] = j / G
__global__ __launch_bounds__(256) void act_order_index_kernel(const int32_t* __restrict__ perm, uint32_t K, int G,
                                                              int32_t* __restrict__ g_idx) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t j = blockIdx.x * blockDim.x + threadIdx.x; j < K; j += stride)
    g_idx[clamp_idx(perm[j], K)] = (int32_t)(j / (uint32_t)G);
}

template <typename TW> __device__ __forceinline__ float act_widen(TW v);
template <> __device__ __forceinline__ float act_widen<uint16_t>(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
template <> __device__ __forceinline__ float act_widen<float>(float v) { return v; }

// Per (row, group): the page's scale and zero point over the group's channels. A block
// takes one row into LDS; G/8 lanes read 8 positions of the channel order each, gather
// those channels from LDS and reduce over the group (DPP). The gathers are random within
// the row, so LDS bank conflicts bound this kernel. Sym: s = max(amax / 8, 1e-9); asym:
// s = max(max - min, 1e-9) / 15, zp = clamp(rint(-min / s), 0, 15).
template <bool SYM, int G, typename TW>
__global__ __launch_bounds__(kParamThreads) void act_order_params_kernel(const TW* __restrict__ W, int64_t ldw,
                                                               const int32_t* __restrict__ perm, int N, int K,
                                                               float* __restrict__ ps, uint8_t* __restrict__ pz) {
  constexpr int LG = G / 8;                     // lanes per group
  constexpr int E16 = 16 / sizeof(TW);          // elements per 16-byte chunk
  extern __shared__ uint32_t lds[];
  TW* row = reinterpret_cast<TW*>(lds);         // [K]
  const int t = threadIdx.x, NG = K / G, i = t % LG, n = blockIdx.x;
  stage16<kParamThreads>(reinterpret_cast<U4*>(row), reinterpret_cast<const U4*>(W + (int64_t)n * ldw), K / E16);
  __syncthreads();
  for (int g = t / LG; g < NG; g += kParamThreads / LG) {     // the same for the LG lanes of a group
    const int j = g * G + 8 * i;
    const U4 pa = ld16(perm + j), pb = ld16(perm + j + 4);
    const uint32_t pj[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float x = act_widen<TW>(row[clamp_idx((int32_t)pj[q], (uint32_t)K)]);
      if constexpr (SYM) {
        hi = q ? fmaxf(hi, fabsf(x)) : fabsf(x);
      } else {
        lo = q ? fminf(lo, x) : x;
        hi = q ? fmaxf(hi, x) : x;
      }
    }
    hi = lanes_max<LG>(hi);
    if constexpr (!SYM) lo = lanes_min<LG>(lo);
    if (i == 0) {
      if constexpr (SYM) {
        ps[(int64_t)n * NG + g] = fmaxf(hi * 0.125f, 1e-9f);   // amax / 8: exact scaling by 2^-3
      } else {
        const float sc = fmaxf(hi - lo, 1e-9f) / 15.0f;
        ps[(int64_t)n * NG + g] = sc;
        pz[(int64_t)n * NG + g] = (uint8_t)__builtin_amdgcn_fmed3f(rintf(-lo / sc), 0.0f, 15.0f);
      }
    }
  }
}

// Codes in channel order, tile layout of gptq.hip: wave w holds rows 8w..8w+7, lane l
// holds k = k0 + 8l..8l+7; code = clamp(rint(x / s) + zp, 0, 15) with (s, zp) of group
// g_idx[k]. The k-tile 0 of each row band also writes the band's fp16 scales and qzeros.
// LDS holds one word per (group, row): y = rcp(s) (within 1 ulp of 1/s) with its low 4
// mantissa bits replaced by the zero point (asymmetric), a relative change below 2^-19.
// For u = fma(x, y, zp) in [-1, 16] the quotient t = x / s has |t| <= 32, so
// |u - (t + zp)| <= 32 * (2^-23 + 2^-19) + 2^-20 and |fl(x / s) - t| <= 32 * 2^-24: u is
// within 2^-13 of v = fl(x / s) + zp, and when |u - rint(u)| < 0.5 - 2^-12 the page's
// rint(v) equals rint(u). Beyond that range the clamp gives the same code for u and v
// (u > 16: v > 15.5; u < -1: v < -0.5). Weights that fail the margin (ties and near ties)
// divide exactly, wherever u lies.
template <bool SYM, typename TW>
__global__ __launch_bounds__(256) void act_order_codes_kernel(const TW* __restrict__ W, int64_t ldw,
                                                              const int32_t* __restrict__ g_idx,
                                                              const float* __restrict__ ps,
                                                              const uint8_t* __restrict__ pz, int N, int K, int NG,
                                                              int ntk, uint32_t* __restrict__ qweight,
                                                              _Float16* __restrict__ scales,
                                                              uint32_t* __restrict__ qzeros) {
  extern __shared__ uint32_t lds[];
  uint32_t* qtile = lds;                                              // [kTR][kQS]
  uint32_t* ytile = lds + kTR * kQS;                                  // [NG][kPS] rcp(s) | zp
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int nt = blockIdx.x / ntk, kt = blockIdx.x - nt * ntk;
  const int n0 = nt * kTN, k0 = kt * kTK;
  // lanes past K and rows past N read valid places; nothing of theirs reaches memory
  const int kc = min(k0 + lane * 8, K - 8);
  Raw8<TW> raw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) raw[i] = load_raw8(W + (int64_t)min(n0 + wave * 8 + i, N - 1) * ldw + kc);
  uint32_t gi[8];
  {
    const U4 ga = ld16(g_idx + kc), gb = ld16(g_idx + kc + 4);
    const uint32_t g8[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) gi[j] = clamp_idx((int32_t)g8[j], (uint32_t)NG);
  }
  // the band's parameters are one contiguous run of ps / pz ([N][NG]); rows past N
  // repeat row N - 1
  for (int e0 = t; e0 < NG * kTN; e0 += 256 * kBatch) {
    float sv[kBatch];
    uint8_t zv[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int e = e0 + 256 * q;
      if (e < NG * kTN) {
        const int rl = e / NG;
        const int64_t at = (int64_t)min(n0 + rl, N - 1) * NG + (e - rl * NG);
        sv[q] = ps[at];
        if constexpr (!SYM) zv[q] = pz[at];
      }
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int e = e0 + 256 * q;
      if (e < NG * kTN) {
        const int rl = e / NG, g = e - rl * NG;
        const uint32_t y = __float_as_uint(__builtin_amdgcn_rcpf(sv[q]));
        ytile[g * kPS + rl] = SYM ? y : ((y & ~0xFu) | zv[q]);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rl = wave * 8 + i;
    float x[8];
    to_f32(raw[i], x);
    uint32_t ev = 0, od = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t yw = ytile[gi[j] * kPS + rl];
      const float zp = SYM ? 8.0f : (float)(yw & 0xFu);
      const float u = __builtin_fmaf(x[j], __uint_as_float(yw), zp);
      float c = rintf(u);
      if (fabsf(u - c) >= 0.5f - 0x1p-12f) {
        const float sc = ps[(int64_t)min(n0 + rl, N - 1) * NG + gi[j]];
        c = rintf(x[j] / sc) + zp;
      }
      c = __builtin_amdgcn_fmed3f(c, 0.0f, 15.0f);
      if (j & 1) od = __builtin_amdgcn_cvt_pk_u8_f32(c, j >> 1, od);
      else ev = __builtin_amdgcn_cvt_pk_u8_f32(c, j >> 1, ev);
    }
    qtile[lane * kQS + rl] = ev | (od << 4);
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
  if (kt == 0) {
    for (int e = t; e < NG * kTN; e += 256) {     // scales [K/G, N]
      const int g = e / kTN, rl = e - g * kTN;
      if (n0 + rl < N) scales[(int64_t)g * N + n0 + rl] = (_Float16)ps[(int64_t)(n0 + rl) * NG + g];
    }
    for (int e = t; e < NG * (kTN / 8); e += 256) {   // qzeros [K/G, N/8]
      const int g = e / (kTN / 8), q = e - g * (kTN / 8);
      if (n0 + 8 * q < N) {
        uint32_t w = 0x77777777u;
        if constexpr (!SYM) {
          w = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) w |= (ytile[g * kPS + 8 * q + i] & 0xFu) << (4 * i);
        }
        qzeros[(int64_t)g * (N / 8) + n0 / 8 + q] = w;
      }
    }
  }
}

// Dequantize (SINK kStore) or accumulate the error against W (SINK kErr) with per-channel
// groups. The tile layout follows gptq_dequant_kernel: wave w holds rows 8w..8w+7 of the
// 32-row tile, lane l holds k = k0 + 8l..8l+7. LDS: the qweight tile, then every group's
// scale (fp16 widened to float32) and zero point for the 32 rows, [group][kPS].
template <int SINK, bool SYM, typename TOut, typename TW>
__global__ __launch_bounds__(256) void gptq_act_dequant_kernel(const uint32_t* __restrict__ qweight,
                                                               const _Float16* __restrict__ scales,
                                                               const uint32_t* __restrict__ qzeros,
                                                               const int32_t* __restrict__ g_idx, int N, int K,
                                                               int NG, int ntk, int ntiles, TOut* __restrict__ out,
                                                               int64_t ldo, const TW* __restrict__ W, int64_t ldw,
                                                               double* __restrict__ part) {
  extern __shared__ uint32_t lds[];
  uint32_t* qtile = lds;                                            // [kTR][kQS]
  float* stile = reinterpret_cast<float*>(lds + kTR * kQS);         // [NG][kPS]
  uint8_t* ztile = reinterpret_cast<uint8_t*>(stile + NG * kPS);    // [NG][kPS]
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  double sw = 0.0, se = 0.0;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int nt = tile / ntk, kt = tile - nt * ntk;
    const int n0 = nt * kTN, k0 = kt * kTK;
    const int r = t >> 2, c8 = (t & 3) * 8;
    const bool qok = k0 / 8 + r < K / 8 && n0 + c8 < N;
    U4 qa{}, qb{};
    if (qok) {
      const uint32_t* src = qweight + (int64_t)(k0 / 8 + r) * N + n0 + c8;
      qa = ld16(src);
      qb = ld16(src + 4);
    }
    const int k = k0 + lane * 8;
    uint32_t gi[8];
    if (k < K) {
      const U4 ga = ld16(g_idx + k), gb = ld16(g_idx + k + 4);
      const uint32_t g8[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) gi[j] = clamp_idx((int32_t)g8[j], (uint32_t)NG);
    }
    Raw8<TW> wr[8];
    if constexpr (SINK == kErr) {
      const int kc = min(k, K - 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) wr[i] = load_raw8(W + (int64_t)min(n0 + wave * 8 + i, N - 1) * ldw + kc);
    }
    for (int e = t; e < NG * kTN; e += 256) {
      const int g = e / kTN, rl = e - g * kTN;
      const int n = min(n0 + rl, N - 1);
      stile[g * kPS + rl] = (float)scales[(int64_t)g * N + n];
      if constexpr (!SYM) ztile[g * kPS + rl] = (uint8_t)((qzeros[(int64_t)g * (N / 8) + n / 8] >> (4 * (n % 8))) & 0xFu);
    }
    if (qok) {
      uint32_t* dst = &qtile[r * kQS + c8];
      dst[0] = qa.x; dst[1] = qa.y; dst[2] = qa.z; dst[3] = qa.w;
      dst[4] = qb.x; dst[5] = qb.y; dst[6] = qb.z; dst[7] = qb.w;
    }
    __syncthreads();
    if (k < K) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rl = wave * 8 + i;
        const int n = n0 + rl;
        if (n < N) {
          const uint32_t word = qtile[lane * kQS + rl];
          float d[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float s = stile[gi[j] * kPS + rl];
            const float z = SYM ? 8.0f : (float)ztile[gi[j] * kPS + rl];
            // (c - z) * s: the page's float ops; exact in float32 for a finite fp16 scale
            d[j] = ((float)((word >> (4 * j)) & 0xFu) - z) * s;
          }
          if constexpr (SINK == kStore) {
            store8(out + (int64_t)n * ldo + k, d);
          } else {
            float x[8];
            to_f32(wr[i], x);
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
static int act_ntk(int64_t K) { return (int)((K + kTK - 1) / kTK); }
static unsigned act_tiles(int64_t N, int64_t K) { return (unsigned)(((N + kTN - 1) / kTN) * act_ntk(K)); }
static size_t act_lds_bytes(int NG) {
  return sizeof(uint32_t) * (size_t)kTR * kQS + (size_t)NG * kPS * (sizeof(float) + 1);
}
static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t gptq_act_workspace_bytes(int64_t N, int64_t K, int group) {
  const size_t pairs = (size_t)N * (size_t)(K / group);
  return align256(pairs * 4) + align256(pairs);              // float32 scales, zero points
}

template <bool SYM, int G, typename TW>
static void act_params_launch(const void* W, int64_t N, int64_t K, int64_t ldw, const int32_t* perm, float* ps,
                              uint8_t* pz, hipStream_t st) {
  hipLaunchKernelGGL((act_order_params_kernel<SYM, G, TW>), dim3((unsigned)N), dim3(kParamThreads), (size_t)K * sizeof(TW), st,
                     (const TW*)W, ldw, perm, (int)N, (int)K, ps, pz);
}
template <bool SYM, typename TW>
static void act_quant_t(int group, const void* W, int64_t N, int64_t K, int64_t ldw, const int32_t* perm,
                        void* qweight, void* scales, void* qzeros, int32_t* g_idx, void* workspace, hipStream_t st) {
  const int NG = (int)(K / group);
  float* ps = (float*)workspace;
  uint8_t* pz = (uint8_t*)workspace + align256((size_t)N * NG * 4);
  hipLaunchKernelGGL(act_order_index_kernel, dim3(stream_blocks((uint64_t)K)), dim3(256), 0, st, perm, (uint32_t)K,
                     group, g_idx);
  if (group == 32) act_params_launch<SYM, 32, TW>(W, N, K, ldw, perm, ps, pz, st);
  else if (group == 64) act_params_launch<SYM, 64, TW>(W, N, K, ldw, perm, ps, pz, st);
  else act_params_launch<SYM, 128, TW>(W, N, K, ldw, perm, ps, pz, st);
  const size_t lds = sizeof(uint32_t) * ((size_t)kTR * kQS + (size_t)NG * kPS);
  hipLaunchKernelGGL((act_order_codes_kernel<SYM, TW>), dim3(act_tiles(N, K)), dim3(256), lds, st, (const TW*)W, ldw,
                     (const int32_t*)g_idx, (const float*)ps, (const uint8_t*)pz, (int)N, (int)K, NG, act_ntk(K),
                     (uint32_t*)qweight, (_Float16*)scales, (uint32_t*)qzeros);
}

void launch_gptq_act_quant(bool sym, int group, const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw,
                           const int32_t* perm, void* qweight, void* scales, void* qzeros, int32_t* g_idx,
                           void* workspace, hipStream_t st) {
  if (sym) {
    if (w_dtype == kBF16) act_quant_t<true, uint16_t>(group, W, N, K, ldw, perm, qweight, scales, qzeros, g_idx, workspace, st);
    else act_quant_t<true, float>(group, W, N, K, ldw, perm, qweight, scales, qzeros, g_idx, workspace, st);
  } else {
    if (w_dtype == kBF16) act_quant_t<false, uint16_t>(group, W, N, K, ldw, perm, qweight, scales, qzeros, g_idx, workspace, st);
    else act_quant_t<false, float>(group, W, N, K, ldw, perm, qweight, scales, qzeros, g_idx, workspace, st);
  }
}

template <int SINK, bool SYM, typename TOut, typename TW>
static void act_deq_launch(unsigned grid, int group, const void* qw, const void* sc, const void* qz,
                           const int32_t* g_idx, int64_t N, int64_t K, void* out, int64_t ldo, const void* W,
                           int64_t ldw, double* part, hipStream_t st) {
  const int NG = (int)(K / group);
  hipLaunchKernelGGL((gptq_act_dequant_kernel<SINK, SYM, TOut, TW>), dim3(grid), dim3(256), act_lds_bytes(NG),
                     st, (const uint32_t*)qw, (const _Float16*)sc, (const uint32_t*)qz, g_idx, (int)N, (int)K, NG,
                     act_ntk(K), (int)act_tiles(N, K), (TOut*)out, ldo, (const TW*)W, ldw, part);
}

void launch_gptq_act_dequant(bool sym, int group, const void* qweight, const void* scales, const void* qzeros,
                             const int32_t* g_idx, int64_t N, int64_t K, void* out, int32_t out_dtype, int64_t ldo,
                             hipStream_t st) {
  const unsigned grid = act_tiles(N, K);
  if (sym) {
    if (out_dtype == kBF16)
      act_deq_launch<kStore, true, uint16_t, uint16_t>(grid, group, qweight, scales, qzeros, g_idx, N, K, out, ldo,
                                                       nullptr, 0, nullptr, st);
    else
      act_deq_launch<kStore, true, float, uint16_t>(grid, group, qweight, scales, qzeros, g_idx, N, K, out, ldo,
                                                    nullptr, 0, nullptr, st);
  } else {
    if (out_dtype == kBF16)
      act_deq_launch<kStore, false, uint16_t, uint16_t>(grid, group, qweight, scales, qzeros, g_idx, N, K, out, ldo,
                                                        nullptr, 0, nullptr, st);
    else
      act_deq_launch<kStore, false, float, uint16_t>(grid, group, qweight, scales, qzeros, g_idx, N, K, out, ldo,
                                                     nullptr, 0, nullptr, st);
  }
}

unsigned gptq_act_err_blocks(int64_t N, int64_t K) {
  const unsigned t = act_tiles(N, K);
  const unsigned cap = 16 * kErrGridCap;
  return t < cap ? (t ? t : 1) : cap;
}

void launch_gptq_act_err(bool sym, int group, const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw,
                         const void* qweight, const void* scales, const void* qzeros, const int32_t* g_idx,
                         double* part, hipStream_t st) {
  const unsigned grid = gptq_act_err_blocks(N, K);
  if (sym) {
    if (w_dtype == kBF16)
      act_deq_launch<kErr, true, float, uint16_t>(grid, group, qweight, scales, qzeros, g_idx, N, K, nullptr, 0, W,
                                                  ldw, part, st);
    else
      act_deq_launch<kErr, true, float, float>(grid, group, qweight, scales, qzeros, g_idx, N, K, nullptr, 0, W, ldw,
                                               part, st);
  } else {
    if (w_dtype == kBF16)
      act_deq_launch<kErr, false, float, uint16_t>(grid, group, qweight, scales, qzeros, g_idx, N, K, nullptr, 0, W,
                                                   ldw, part, st);
    else
      act_deq_launch<kErr, false, float, float>(grid, group, qweight, scales, qzeros, g_idx, N, K, nullptr, 0, W,
                                                ldw, part, st);
  }
}

// ------------------------------------------------------------- group order
// Act-order tensors rearranged for the decode GEMV, once per weight: the channels taken
// group by group, ascending inside a group, so group g's channels sit at positions
// g*G .. g*G + G - 1 and the index-order GPTQ kernels apply to the gathered activations.
// perm: thread g scans g_idx in channel order and places its group's channels; a group
// of another size, or a group index outside [0, K/G), sets the status word (1: a group
// does not hold exactly G channels, 2: g_idx out of range; 0: none).
__global__ __launch_bounds__(256) void gptq_group_perm_kernel(const int32_t* __restrict__ g_idx, int K, int G, int NG,
                                                              int32_t* __restrict__ perm, int32_t* __restrict__ status) {
  const int g = threadIdx.x;
  int sizes_bad = 0, range_bad = 0;
  if (g < NG) {
    int cnt = 0;
    for (int k = 0; k < K; ++k) {
      if (g_idx[k] == g) {
        if (cnt < G) perm[g * G + cnt] = k;
        ++cnt;
      }
    }
    sizes_bad = cnt != G;
  }
  for (int k = threadIdx.x; k < K; k += 256) {
    const int gk = g_idx[k];
    range_bad |= gk < 0 || gk >= NG;
  }
  const int rb = __syncthreads_or(range_bad), sb = __syncthreads_or(sizes_bad);
  if (threadIdx.x == 0) *status = rb ? 2 : (sb ? 1 : 0);
}

// Word (r, n) of the rearranged qweight: nibble i = code of channel perm[8r + i]. perm
// entries are clamped into [0, K): a refused g_idx leaves unwritten slots, whose reads
// stay in bounds (the status word reports the refusal).
__global__ __launch_bounds__(256) void gptq_group_repack_kernel(const uint32_t* __restrict__ qweight, int N, int K,
                                                                const int32_t* __restrict__ perm,
                                                                uint32_t* __restrict__ out) {
  const int n = blockIdx.x * 256 + threadIdx.x, r = blockIdx.y;
  if (n >= N) return;
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k = min(max(perm[8 * r + i], 0), K - 1);
    const uint32_t src = qweight[(int64_t)(k >> 3) * N + n];
    w |= ((src >> (4 * (k & 7))) & 0xFu) << (4 * i);
  }
  out[(int64_t)r * N + n] = w;
}

void launch_gptq_group_order(int group, const void* qweight, const int32_t* g_idx, int64_t N, int64_t K,
                             void* qweight_out, int32_t* perm, int32_t* status, hipStream_t st) {
  const int NG = (int)(K / group);                               // <= kActMaxGroups: one thread per group
  hipLaunchKernelGGL(gptq_group_perm_kernel, dim3(1), dim3(256), 0, st, g_idx, (int)K, group, NG, perm, status);
  hipLaunchKernelGGL(gptq_group_repack_kernel, dim3((unsigned)((N + 255) / 256), (unsigned)(K / 8)), dim3(256), 0, st,
                     (const uint32_t*)qweight, (int)N, (int)K, perm, (uint32_t*)qweight_out);
}

// The activations gathered into group order: xo[b][j] = x[b][perm[j]] (perm clamped into
// [0, K)), rows of K contiguous.
__global__ __launch_bounds__(256) void gather_columns_kernel(const uint16_t* __restrict__ x, int64_t ldx, int B, int K,
                                                             const int32_t* __restrict__ perm,
                                                             uint16_t* __restrict__ xo) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)B * K) return;
  const int b = (int)(e / K), j = (int)(e - (int64_t)b * K);
  const int k = min(max(perm[j], 0), K - 1);
  xo[e] = x[(int64_t)b * ldx + k];
}

void launch_gather_columns(const void* x, int64_t ldx, int64_t B, int64_t K, const int32_t* perm, void* xo,
                           hipStream_t st) {
  const int64_t total = B * K;
  hipLaunchKernelGGL(gather_columns_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                     (const uint16_t*)x, ldx, (int)B, (int)K, perm, (uint16_t*)xo);
}

}  // namespace gwb
