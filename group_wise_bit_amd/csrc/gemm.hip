// Prefill GEMM on quantized weights: y[m, n] = sum_k x[m, k] * dequant(W)[n, k] for M
// rows of bf16 activations. Page export_gptq_cpu.py: vLLM's W4A16 kernels consume the
// GPTQ tensors as stored; page quantize_dflash_mxfp4.py serves its linears as MXFP4.
// The dequantized weights never reach memory: each wavefront turns its packed words
// into bf16 B operands of the matrix cores (v_mfma_f32_16x16x32_bf16, float32
// accumulation) in registers, and the activations are staged through LDS, shared by
// the block's four wavefronts.
//
// Block: 4 wavefronts, BM = 16*MT rows x 256 columns; wavefront w owns columns
// n0 + 64w .. +63 and all BM rows (MT x 4 MFMA tiles of 16 x 16). Lane l (j = l % 16,
// q = l / 16) feeds B column j of tile t with the weights of column nb + 4j + t, so its
// accumulators hold rows 16mt + 4q + r (r < 4) of the 4 adjacent columns nb + 4j .. +3.
// K runs in stages of 128 through a double-buffered LDS tile of activations.
//
// GPTQ: codes c are integers and bf16(128 + c) is exact; (w >> 4i) & 0x000F000F |
// 0x43004300 gives codes i and i + 4 of a word as such a pair. Per group the matrix
// cores sum T = sum_k x (128 + c) (exact products); the group adds
// s * (T - (128 + z) * sum_k x) to the output, with the group sums of x from a pre-pass
// (float64 sums, rounded once). The activations sit in LDS in the pairs' within-8 order
// (k = 0, 4, 1, 5, 2, 6, 3, 7). A step covers 32 consecutive k, so a group ends on a
// step boundary for every group size.
// MXFP4: the scaled FP4 conversion gives the exact bf16 weights (E2M1 times
// 2^(e8m0 - 127)). A lane's 8-k slot in step s is k0 + 32q + 8s, so over a stage it
// covers one 32-block of each of its columns: one 16-byte load of codes and one scale
// byte per column and stage.
#include "kernels.hpp"
#include "mxfp4_math.hpp"

namespace gwb {

typedef __bf16 gm_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float gm_f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGmBN = 256;            // columns per block
constexpr int kGmBK = 128;            // k per stage
constexpr int kGmLd = kGmBK + 8;      // LDS row stride of the activation tile (bf16)
constexpr int kGmSumMax = 4 * 128;    // group sums of one stage: up to 4 groups x BM rows

__device__ __forceinline__ gm_f32x4_t mfma_bf16(U4 a, U4 b, gm_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gm_bf16x8_t, a),
                                                  __builtin_bit_cast(gm_bf16x8_t, b), c, 0, 0, 0);
}

// Workgroups go round-robin over the 8 XCDs, each with its own L2. Each XCD gets a
// contiguous range of tiles; tiles run in bands of up to 4 row tiles across all column
// tiles, so the blocks an XCD holds at one time share activation rows and weights.
__device__ __forceinline__ void gemm_tile(int gx, int gy, int& bx, int& by) {
  const int T = gx * gy, id = blockIdx.x, xcd = id & 7, rem = T & 7;
  const int t = xcd * (T >> 3) + min(xcd, rem) + (id >> 3);
  const int band = t / (4 * gy), first = band * 4, rows = min(4, gx - first);
  const int r = t - first * gy;
  bx = first + r % rows;
  by = r / rows;
}

// Block-cooperative copy of the activation tile rows m0 .. m0+BM-1, k0 .. k0+127:
// chunk c = thread + 256 i is row c / 16, 8-k slot c % 16 (rows past M read as 0).
template <int MT>
__device__ __forceinline__ void a_load(const uint16_t* __restrict__ x, int64_t ldx, int M, int m0, int k0,
                                       U4 (&v)[MT]) {
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int c = (int)threadIdx.x + 256 * i, m = m0 + (c >> 4);
    v[i] = m < M ? ld16(x + (int64_t)m * ldx + k0 + 8 * (c & 15)) : U4{0u, 0u, 0u, 0u};
  }
}
// PAIRS: store each 8-k slot as (x0, x4), (x1, x5), (x2, x6), (x3, x7).
template <int MT, bool PAIRS>
__device__ __forceinline__ void a_store(uint16_t* lds, const U4 (&v)[MT]) {
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int c = (int)threadIdx.x + 256 * i;
    U4 u = v[i];
    if constexpr (PAIRS)
      u = U4{__builtin_amdgcn_perm(u.z, u.x, 0x05040100u), __builtin_amdgcn_perm(u.z, u.x, 0x07060302u),
             __builtin_amdgcn_perm(u.w, u.y, 0x05040100u), __builtin_amdgcn_perm(u.w, u.y, 0x07060302u)};
    st16(lds + (c >> 4) * kGmLd + 8 * (c & 15), u);
  }
}

// Rows 16mt + 4q + r of the lane's 4 columns nl .. nl+3.
template <int MT, typename TY>
__device__ __forceinline__ void gemm_store(const gm_f32x4_t (&acc)[MT][4], TY* __restrict__ y, int64_t ldy, int M,
                                           int m0, int q, int nl, bool nok) {
  if (!nok) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 16 * mt + 4 * q + r;
      if (m >= M) continue;
      TY* p = y + (int64_t)m * ldy + nl;
      if constexpr (sizeof(TY) == 4) {
        *reinterpret_cast<float4*>(p) = float4{acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]};
      } else {
        *reinterpret_cast<uint2*>(p) =
            uint2{pack_bf16x2(acc[mt][0][r], acc[mt][1][r]), pack_bf16x2(acc[mt][2][r], acc[mt][3][r])};
      }
    }
}

// ------------------------------------------------------------------ group sums
// sums[g * Mp + m] = sum of x[m, gG .. gG+G-1] in float64, rounded once to float32;
// rows M .. Mp-1 get 0. One lane per 8 activations, G/8 lanes (aligned) per group.
template <int G>
__global__ __launch_bounds__(256) void gemm_group_sums_kernel(const uint16_t* __restrict__ x, int64_t ldx, int M,
                                                             int K, int Mp, float* __restrict__ sums) {
  constexpr int L = G / 8;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x, per_row = K / 8;
  const bool live = id < (int64_t)Mp * per_row;
  int m = 0, kc = 0;
  double s = 0.0;
  if (live) {
    m = (int)(id / per_row);
    kc = (int)(id - (int64_t)m * per_row);
    if (m < M) {
      const U4 v = ld16(x + (int64_t)m * ldx + 8 * kc);
      s = ((double)bf16_lo(v.x) + (double)bf16_hi(v.x)) + ((double)bf16_lo(v.y) + (double)bf16_hi(v.y)) +
          (((double)bf16_lo(v.z) + (double)bf16_hi(v.z)) + ((double)bf16_lo(v.w) + (double)bf16_hi(v.w)));
    }
  }
#pragma unroll
  for (int o = 1; o < L; o <<= 1) s += __shfl_xor(s, o);
  if (live && kc % L == 0) sums[(int64_t)(kc / L) * Mp + m] = (float)s;
}

// ------------------------------------------------------------------ GPTQ
template <bool SYM, int G, int MT, typename TY>
__global__ __launch_bounds__(256, 1) void gptq_gemm_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int M, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ sc, const uint32_t* __restrict__ qz, int N, int K, const float* __restrict__ gsum,
    int Mp, TY* __restrict__ y, int64_t ldy, int gx, int gy) {
  constexpr int BM = 16 * MT, SPG = G / 32, NGS = kGmBK / G;   // steps per group, groups per stage
  constexpr int SUMS = BM * NGS / 4;                            // float4 chunks of group sums per stage
  static_assert(SUMS <= 256 && BM * NGS <= kGmSumMax, "group sums of a stage fit one chunk per thread");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kGmLd];
  __shared__ __attribute__((aligned(16))) float Ss[2][NGS * BM];

  int bx, by;
  gemm_tile(gx, gy, bx, by);
  const int lane = threadIdx.x & 63, j = lane & 15, q = lane >> 4;
  const int m0 = bx * BM, nl = by * kGmBN + (int)(threadIdx.x >> 6) * 64 + 4 * j;
  const bool nok = nl < N;
  const int tid = threadIdx.x;

  // stage prefetch: activations, group sums, code words, scales and zero points
  U4 av[MT], wv[4];
  float4 sv = float4{0.f, 0.f, 0.f, 0.f};
  uint2 scv[NGS];
  uint32_t zv[NGS];
  auto fetch = [&](int k0) {
    a_load<MT>(x, ldx, M, m0, k0, av);
    if (tid < SUMS) {
      const int gi = tid / (BM / 4), rr = 4 * (tid % (BM / 4));
      sv = *reinterpret_cast<const float4*>(gsum + (int64_t)(k0 / G + gi) * Mp + m0 + rr);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
      wv[s] = nok ? ld16(qw + (int64_t)(k0 / 8 + 4 * s + q) * N + nl) : U4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int gi = 0; gi < NGS; ++gi) {
      const int g = k0 / G + gi;
      scv[gi] = nok ? *reinterpret_cast<const uint2*>(sc + (int64_t)g * N + nl) : uint2{0u, 0u};
      if constexpr (!SYM) zv[gi] = nok ? qz[(int64_t)g * (N / 8) + nl / 8] : 0u;
    }
  };
  auto commit = [&](int buf) {
    a_store<MT, true>(As[buf], av);
    if (tid < SUMS) *reinterpret_cast<float4*>(&Ss[buf][4 * tid]) = sv;
  };

  gm_f32x4_t acc[MT][4], tmp[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[mt][t] = gm_f32x4_t{0.f, 0.f, 0.f, 0.f};

  fetch(0);
  commit(0);
  __syncthreads();
  const int nst = K / kGmBK;
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    const uint16_t* A = As[buf] + j * kGmLd + 8 * q;
    U4 w[4];
    uint2 scl[NGS];
    uint32_t zl[NGS];
#pragma unroll
    for (int s = 0; s < 4; ++s) w[s] = wv[s];
#pragma unroll
    for (int gi = 0; gi < NGS; ++gi) {
      scl[gi] = scv[gi];
      if constexpr (!SYM) zl[gi] = zv[gi];
    }
    if (st + 1 < nst) fetch((st + 1) * kGmBK);

#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t wd[4] = {w[s].x, w[s].y, w[s].z, w[s].w};
      U4 b[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        b[t] = U4{(wd[t] & 0x000F000Fu) | 0x43004300u, ((wd[t] >> 4) & 0x000F000Fu) | 0x43004300u,
                  ((wd[t] >> 8) & 0x000F000Fu) | 0x43004300u, ((wd[t] >> 12) & 0x000F000Fu) | 0x43004300u};
      if (s % SPG == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int t = 0; t < 4; ++t) tmp[mt][t] = gm_f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const U4 a = *reinterpret_cast<const U4*>(A + 16 * mt * kGmLd + 32 * s);
#pragma unroll
        for (int t = 0; t < 4; ++t) tmp[mt][t] = mfma_bf16(a, b[t], tmp[mt][t]);
      }
      if (s % SPG == SPG - 1) {   // the group ends: acc += s * (T - (128 + z) * sum x)
        const int gi = s / SPG;
        const uint32_t sb[4] = {scl[gi].x & 0xFFFFu, scl[gi].x >> 16, scl[gi].y & 0xFFFFu, scl[gi].y >> 16};
        float sf[4], cz[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          sf[t] = (float)__builtin_bit_cast(_Float16, (uint16_t)sb[t]);
          if constexpr (SYM) cz[t] = -136.0f;
          else cz[t] = -(float)(128u + ((zl[gi] >> (4 * ((nl & 7) + t))) & 0xFu));
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const float4 sx = *reinterpret_cast<const float4*>(&Ss[buf][gi * BM + 16 * mt + 4 * q]);
          const float sxa[4] = {sx.x, sx.y, sx.z, sx.w};
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[mt][t][r] = fmaf(sf[t], fmaf(cz[t], sxa[r], tmp[mt][t][r]), acc[mt][t][r]);
        }
      }
    }
    if (st + 1 < nst) commit(buf ^ 1);
    __syncthreads();
  }
  gemm_store<MT, TY>(acc, y, ldy, M, m0, q, nl, nok);
}

// ------------------------------------------------------------------ MXFP4
template <int MT, typename TY>
__global__ __launch_bounds__(256, 1) void mxfp4_gemm_kernel(const uint16_t* __restrict__ x, int64_t ldx, int M,
                                                           const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ e8m0, int N, int K,
                                                           TY* __restrict__ y, int64_t ldy, int gx, int gy) {
  constexpr int BM = 16 * MT;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kGmLd];

  int bx, by;
  gemm_tile(gx, gy, bx, by);
  const int lane = threadIdx.x & 63, j = lane & 15, q = lane >> 4;
  const int m0 = bx * BM, nl = by * kGmBN + (int)(threadIdx.x >> 6) * 64 + 4 * j;
  const bool nok = nl < N;
  const int64_t rowb = K / 2, rows = K / 32;

  U4 av[MT], wv[4];
  uint32_t ev[4];
  auto fetch = [&](int k0) {
    a_load<MT>(x, ldx, M, m0, k0, av);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      wv[t] = nok ? ld16(codes + (int64_t)(nl + t) * rowb + k0 / 2 + 16 * q) : U4{0u, 0u, 0u, 0u};
      ev[t] = nok ? (uint32_t)e8m0[(int64_t)(nl + t) * rows + k0 / 32 + q] : 127u;
    }
  };

  gm_f32x4_t acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[mt][t] = gm_f32x4_t{0.f, 0.f, 0.f, 0.f};

  fetch(0);
  a_store<MT, false>(As[0], av);
  __syncthreads();
  const int nst = K / kGmBK;
  for (int st = 0; st < nst; ++st) {
    const uint16_t* A = As[st & 1] + j * kGmLd + 32 * q;
    U4 w[4];
    uint32_t e[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      w[t] = wv[t];
      e[t] = ev[t];
    }
    if (st + 1 < nst) fetch((st + 1) * kGmBK);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      U4 b[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t wd = s == 0 ? w[t].x : s == 1 ? w[t].y : s == 2 ? w[t].z : w[t].w;
        b[t] = mx_unpack8_bf16(wd, e[t]);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const U4 a = *reinterpret_cast<const U4*>(A + 16 * mt * kGmLd + 8 * s);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[mt][t] = mfma_bf16(a, b[t], acc[mt][t]);
      }
    }
    if (st + 1 < nst) a_store<MT, false>(As[(st & 1) ^ 1], av);
    __syncthreads();
  }
  gemm_store<MT, TY>(acc, y, ldy, M, m0, q, nl, nok);
}

// ------------------------------------------------------------------ launchers
static int gemm_mt(int64_t M) { return M <= 64 ? 4 : 8; }

size_t gemm_workspace_bytes(bool gptq, int group, int64_t M, int64_t K) {
  if (!gptq) return 0;
  const int64_t Mp = (M + 127) / 128 * 128;
  return (size_t)(K / group) * (size_t)Mp * sizeof(float);
}

template <bool SYM, int G, int MT, typename TY>
static void gptq_gemm_go(const void* x, int64_t ldx, int M, const void* qw, const void* sc, const void* qz, int N,
                         int K, const float* gs, int Mp, void* y, int64_t ldy, hipStream_t st) {
  const int gx = (M + 16 * MT - 1) / (16 * MT), gy = (N + kGmBN - 1) / kGmBN;
  hipLaunchKernelGGL((gptq_gemm_kernel<SYM, G, MT, TY>), dim3(gx * gy), dim3(256), 0, st, (const uint16_t*)x, ldx,
                     M, (const uint32_t*)qw, (const uint16_t*)sc, (const uint32_t*)qz, N, K, gs, Mp, (TY*)y, ldy,
                     gx, gy);
}
// 128-row blocks only with one group per stage: with more, the per-group work of
// 128 rows no longer fits the register file.
template <bool SYM, int G, typename TY>
static void gptq_gemm_mt(int mt, const void* x, int64_t ldx, int M, const void* qw, const void* sc, const void* qz,
                         int N, int K, const float* gs, int Mp, void* y, int64_t ldy, hipStream_t st) {
  if constexpr (G == 128) {
    if (mt == 8) return gptq_gemm_go<SYM, G, 8, TY>(x, ldx, M, qw, sc, qz, N, K, gs, Mp, y, ldy, st);
  }
  gptq_gemm_go<SYM, G, 4, TY>(x, ldx, M, qw, sc, qz, N, K, gs, Mp, y, ldy, st);
}
template <bool SYM, int G>
static void gptq_gemm_ty(int ty, int mt, const void* x, int64_t ldx, int M, const void* qw, const void* sc,
                         const void* qz, int N, int K, const float* gs, int Mp, void* y, int64_t ldy,
                         hipStream_t st) {
  if (ty == GemvOut::kBF16) gptq_gemm_mt<SYM, G, uint16_t>(mt, x, ldx, M, qw, sc, qz, N, K, gs, Mp, y, ldy, st);
  else gptq_gemm_mt<SYM, G, float>(mt, x, ldx, M, qw, sc, qz, N, K, gs, Mp, y, ldy, st);
}
template <int G>
static void group_sums_go(const void* x, int64_t ldx, int M, int K, int Mp, float* sums, hipStream_t st) {
  const int64_t lanes = (int64_t)Mp * (K / 8);
  hipLaunchKernelGGL((gemm_group_sums_kernel<G>), dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, st,
                     (const uint16_t*)x, ldx, M, K, Mp, sums);
}

void launch_gptq_gemm(bool sym, int group, const void* qweight, const void* scales, const void* qzeros, int64_t N,
                      int64_t K, const void* x, int64_t M, int64_t ldx, void* y, int32_t y_dtype, int64_t ldy,
                      float* sums, hipStream_t st) {
  const int Mp = (int)((M + 127) / 128 * 128), mt = gemm_mt(M);
  const int ty = y_dtype == kF32 ? GemvOut::kF32 : GemvOut::kBF16;
#define GWB_GEMM_G(G)                                                                                               \
  do {                                                                                                              \
    group_sums_go<G>(x, ldx, (int)M, (int)K, Mp, sums, st);                                                         \
    if (sym) gptq_gemm_ty<true, G>(ty, mt, x, ldx, (int)M, qweight, scales, qzeros, (int)N, (int)K, sums, Mp, y,    \
                                   ldy, st);                                                                        \
    else gptq_gemm_ty<false, G>(ty, mt, x, ldx, (int)M, qweight, scales, qzeros, (int)N, (int)K, sums, Mp, y, ldy,  \
                                st);                                                                                \
  } while (0)
  if (group == 32) GWB_GEMM_G(32);
  else if (group == 64) GWB_GEMM_G(64);
  else GWB_GEMM_G(128);
#undef GWB_GEMM_G
}

template <int MT, typename TY>
static void mxfp4_gemm_go(const void* x, int64_t ldx, int M, const void* codes, const void* e8, int N, int K,
                          void* y, int64_t ldy, hipStream_t st) {
  const int gx = (M + 16 * MT - 1) / (16 * MT), gy = (N + kGmBN - 1) / kGmBN;
  hipLaunchKernelGGL((mxfp4_gemm_kernel<MT, TY>), dim3(gx * gy), dim3(256), 0, st, (const uint16_t*)x, ldx, M,
                     (const uint8_t*)codes, (const uint8_t*)e8, N, K, (TY*)y, ldy, gx, gy);
}

void launch_mxfp4_gemm(const void* packed, const void* e8m0, int64_t N, int64_t K, const void* x, int64_t M,
                       int64_t ldx, void* y, int32_t y_dtype, int64_t ldy, hipStream_t st) {
  const int mt = gemm_mt(M);
  if (y_dtype == kF32) {
    if (mt == 4) mxfp4_gemm_go<4, float>(x, ldx, (int)M, packed, e8m0, (int)N, (int)K, y, ldy, st);
    else mxfp4_gemm_go<8, float>(x, ldx, (int)M, packed, e8m0, (int)N, (int)K, y, ldy, st);
  } else {
    if (mt == 4) mxfp4_gemm_go<4, uint16_t>(x, ldx, (int)M, packed, e8m0, (int)N, (int)K, y, ldy, st);
    else mxfp4_gemm_go<8, uint16_t>(x, ldx, (int)M, packed, e8m0, (int)N, (int)K, y, ldy, st);
  }
}

}  // namespace gwb
