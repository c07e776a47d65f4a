// Decode GEMV on quantized weights: y[b, n] = sum_k x[b, k] * dequant(W)[n, k], with the
// weights read in their packed form (about a quarter of the bf16 bytes). Page
// export_gptq_cpu.py: vLLM's W4A16 kernel consumes the GPTQ tensors directly, and the
// 131072 x 2048 lm_head is the largest read of a decode step; page
// quantize_dflash_mxfp4.py serves its linears as MXFP4.
//
// Activations are bf16 [B, K] (B <= 8), results float32 or bf16 [B, N]. Every product
// of a dequantized value and an activation is exact in float32; sums accumulate in
// float32 in a fixed order (deterministic for a given shape).
//
// GPTQ ([K/8, N] words, n contiguous): a lane owns 4 adjacent outputs (one 16-byte load
// per qweight row r), a wavefront 256 outputs x 128 k per step (16 loads in flight); a
// block's four wavefronts take contiguous bands of its K range and are combined through
// LDS. With (c - z) * s per group, sum_k (c - z) s x = s (sum_k c x - z sum_k x): codes
// become floats with v_cvt_f32_ubyte, the group sum of x is a wavefront reduction. When
// N alone gives enough blocks, one block covers all of K and writes y; otherwise K is
// split across blocks, whose partial sums a second kernel adds in order.
//
// MXFP4 ([N, K/2] bytes + E8M0 [N, K/32]): lanes run along K, one 32-block per lane
// and step; the codes of a block become bf16 pairs with the scaled FP4 conversion at
// scale 1 (exact), v_dot2c_f32_bf16 multiplies them with the activation pairs, and the
// block sum is scaled by 2^(e8m0 - 127) (exact). A wavefront takes 8 rows at a time and
// reduces each across its lanes.
#include <atomic>

#include "kernels.hpp"
#include "mxfp4_math.hpp"

namespace gwb {

typedef __bf16 gv_bf16x2_t __attribute__((ext_vector_type(2)));

template <typename TY>
__device__ __forceinline__ void store_y(TY* p, float v) {
  if constexpr (sizeof(TY) == 4) *p = v;
  else *p = (uint16_t)f32_to_bf16_rne(v);
}

// Sum over the 64 lanes of a wavefront, fixed butterfly order; every lane gets it.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_read<kDppXor1>(v);
  v += dpp_read<kDppXor2>(v);
  v += dpp_read<kDppHalfMirror>(v);
  v += dpp_read<kDppMirror>(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// VP values per lane (VP = 8 or 16) -> lane l holds the wavefront sum of value l & (VP - 1).
// Each fold halves the values a lane keeps: the half whose index has the lane's bit set
// stays, the other half goes to the DPP partner, which differs in that bit (ror 8 within
// a 16-lane row: bit 3; half mirror 7 - i: bit 2; then bits 1 and 0); lanes 16 and 32
// apart, which hold the same value, are added last. 2 VP - 2 adds instead of 12 VP.
template <int CTRL, int NV, int VP>
__device__ __forceinline__ void gv_fold(float (&v)[VP], bool up) {
#pragma unroll
  for (int i = 0; i < NV / 2; ++i) {
    const float keep = up ? v[i + NV / 2] : v[i], send = up ? v[i] : v[i + NV / 2];
    v[i] = keep + dpp_read<CTRL>(send);
  }
}
template <int VP>
__device__ __forceinline__ float gv_transposed_sum(float (&v)[VP], int lane) {
  static_assert(VP == 8 || VP == 16, "8 or 16 values");
  if constexpr (VP == 16) gv_fold<kDppRor8, 16>(v, lane & 8);
  gv_fold<kDppHalfMirror, 8>(v, lane & 4);
  gv_fold<kDppXor2, 4>(v, lane & 2);
  gv_fold<kDppXor1, 2>(v, lane & 1);
  float r = v[0];
  if constexpr (VP == 8) r += dpp_read<kDppRor8>(r);
  r += __shfl_xor(r, 16);
  r += __shfl_xor(r, 32);
  return r;
}

// ------------------------------------------------------------------ GPTQ
constexpr int kGqWaveK = 128;

// LN adjacent qweight words (columns) of one row, one load. The 4-word load is
// non-temporal: each packed word is read once per call and should not displace the
// activations and scales from the caches.
template <int LN>
__device__ __forceinline__ void load_words(const uint32_t* p, uint32_t (&w)[LN]) {
  if constexpr (LN == 4) {
    const U4 v = ld16_nt(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (LN == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
    w[0] = *p;
  }
}

// One qweight row (8 k) of a lane's LN columns: cx += c x for the group's rows; its
// first row clears cx, its last adds s (sum c x - z sum x) to acc. A 4-bit code c, read
// as an OCP e4m3 byte, is c * 2^-9 exactly (subnormals and the first binade share one
// spacing), so the scaled FP8 conversion at scale 2^9 turns two code bytes into an
// exact bf16 pair; v_dot2_f32_bf16 multiplies it with the matching activation pair
// (products exact, one float32 accumulation each).
template <bool SYM, int B, int LN, int RG>
__device__ __forceinline__ void gq_row(int r, const uint32_t (&w)[LN], const U4 (&xv)[B], const float (&s)[LN],
                                       const float (&z)[LN], const float (&xs)[B], float (&cx)[B][LN],
                                       float (&acc)[B][LN]) {
  if (r % RG == 0) {
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int j = 0; j < LN; ++j) cx[b][j] = 0.0f;
  }
  if constexpr (B > 2) {
    // wider batches: each code widened on its own (v_cvt_f32_ubyte0..3) and one fma per
    // product, so that the activations stay in the order they were loaded (rearranging
    // them costs more scalar registers than a wavefront has)
    float xk[B][8];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const U4 v = xv[b];
      xk[b][0] = bf16_lo(v.x); xk[b][1] = bf16_hi(v.x); xk[b][2] = bf16_lo(v.y); xk[b][3] = bf16_hi(v.y);
      xk[b][4] = bf16_lo(v.z); xk[b][5] = bf16_hi(v.z); xk[b][6] = bf16_lo(v.w); xk[b][7] = bf16_hi(v.w);
    }
#pragma unroll
    for (int j = 0; j < LN; ++j) {
      uint32_t ev = w[j] & 0x0F0F0F0Fu, od = (w[j] >> 4) & 0x0F0F0F0Fu;
      // opaque to the combiner, so each code converts straight from its byte
      asm volatile("" : "+v"(ev), "+v"(od));
      const float c[8] = {(float)(ev & 0xFFu), (float)(od & 0xFFu), (float)((ev >> 8) & 0xFFu),
                          (float)((od >> 8) & 0xFFu), (float)((ev >> 16) & 0xFFu), (float)((od >> 16) & 0xFFu),
                          (float)(ev >> 24), (float)(od >> 24)};
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int q = 0; q < 8; ++q) cx[b][j] = __builtin_fmaf(c[q], xk[b][q], cx[b][j]);
    }
  } else {
    // activation pairs in the order the code pairs come out: (k0, k2), (k4, k6), (k1, k3), (k5, k7)
    gv_bf16x2_t xq[B][4];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const U4 v = xv[b];
      xq[b][0] = __builtin_bit_cast(gv_bf16x2_t, (v.x & 0xFFFFu) | (v.y << 16));
      xq[b][1] = __builtin_bit_cast(gv_bf16x2_t, (v.z & 0xFFFFu) | (v.w << 16));
      xq[b][2] = __builtin_bit_cast(gv_bf16x2_t, (v.x >> 16) | (v.y & 0xFFFF0000u));
      xq[b][3] = __builtin_bit_cast(gv_bf16x2_t, (v.z >> 16) | (v.w & 0xFFFF0000u));
    }
    const float two9 = 512.0f;
#pragma unroll
    for (int j = 0; j < LN; ++j) {
      const uint32_t ev = w[j] & 0x0F0F0F0Fu, od = (w[j] >> 4) & 0x0F0F0F0Fu;   // codes k0 k2 k4 k6 / k1 k3 k5 k7
      const gv_bf16x2_t c[4] = {__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ev, two9, false),
                                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ev, two9, true),
                                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(od, two9, false),
                                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(od, two9, true)};
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) cx[b][j] = __builtin_amdgcn_fdot2_f32_bf16(c[q], xq[b][q], cx[b][j], false);
    }
  }
  if (r % RG == RG - 1) {
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int j = 0; j < LN; ++j) acc[b][j] = __builtin_fmaf(s[j], __builtin_fmaf(-z[j], xs[b], cx[b][j]), acc[b][j]);
  }
}

// One 128-k step of a wavefront: nr qweight rows (FULL: all 16, known at compile time, so
// no row needs a branch and every load can be issued ahead of the arithmetic).
template <bool SYM, int G, int B, int LN, bool FULL>
__device__ __forceinline__ void gq_step(const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scale_bits,
                                        const uint32_t* __restrict__ qzeros, int N, int K,
                                        const uint16_t* __restrict__ x, int64_t ldx, int Bn, int nc, int lane, int kw,
                                        int nr_, float (&acc)[B][LN]) {
  constexpr int NGS = kGqWaveK / G, RG = G / 8;       // groups per step, qweight rows per group
  constexpr int XR = B == 1 ? 16 : 1;                   // rows of activations fetched together
  const int nr = FULL ? kGqWaveK / 8 : nr_;
  // every load of the step is issued before the first use, the small ones first: the
  // step's scales (and zero points), two activations per lane of each group, then the
  // qweight rows
  uint32_t sb[NGS][LN], zw[NGS], xp[NGS][B];
#pragma unroll
  for (int gi = 0; gi < NGS; ++gi) {
    const int g = min(kw + gi * G, K - G) / G;        // groups past K are not used
#pragma unroll
    for (int j = 0; j < LN; ++j) sb[gi][j] = scale_bits[(int64_t)g * N + nc + j];
    zw[gi] = 0u;
    if constexpr (!SYM) zw[gi] = qzeros[(int64_t)g * (N / 8) + nc / 8] >> (4 * (nc % 8));
#pragma unroll
    for (int b = 0; b < B; ++b)
      xp[gi][b] = 2 * lane < G ? *reinterpret_cast<const uint32_t*>(x + (int64_t)min(b, Bn - 1) * ldx + g * G + 2 * lane)
                               : 0u;
  }
  uint32_t wv[kGqWaveK / 8][LN];                      // rows past nr re-read row nr - 1, unused
#pragma unroll
  for (int r = 0; r < kGqWaveK / 8; ++r) load_words<LN>(qweight + (int64_t)(kw / 8 + min(r, nr - 1)) * N + nc, wv[r]);
  __builtin_amdgcn_sched_barrier(0);                 // keep the loads ahead of the arithmetic
  float s[NGS][LN], z[NGS][LN], xs[NGS][B];
#pragma unroll
  for (int gi = 0; gi < NGS; ++gi) {
#pragma unroll
    for (int j = 0; j < LN; ++j) {
      s[gi][j] = (float)__builtin_bit_cast(_Float16, (uint16_t)sb[gi][j]);
      z[gi][j] = SYM ? 8.0f : (float)((zw[gi] >> (4 * j)) & 0xFu);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) xs[gi][b] = wave_sum(bf16_lo(xp[gi][b]) + bf16_hi(xp[gi][b]));
  }
  // rows past nr (a multiple of RG) are skipped by wave-uniform branches, not loop exits:
  // the loops unroll fully and wv stays in registers
  float cx[B][LN];
#pragma unroll
  for (int rc = 0; rc < kGqWaveK / 8; rc += XR) {
    if (rc < nr) {
      U4 xv[XR][B];                                   // the same for every lane
#pragma unroll
      for (int i = 0; i < XR; ++i)
#pragma unroll
        for (int b = 0; b < B; ++b)
          xv[i][b] = *reinterpret_cast<const U4*>(x + (int64_t)min(b, Bn - 1) * ldx + kw + 8 * min(rc + i, nr - 1));
#pragma unroll
      for (int i = 0; i < XR; ++i) {
        const int r = rc + i, gi = r / RG;
        if (r < nr) gq_row<SYM, B, LN, RG>(r, wv[r], xv[i], s[gi], z[gi], xs[gi], cx, acc);
      }
    }
  }
}

// LN: outputs (qweight columns) per lane; a wavefront covers 64 LN of them, and the four
// wavefronts of a block split its K range into contiguous bands of whole 128-k steps,
// combined through LDS in k order. B is the compiled width
// (1, 2, 4, 8); Bn <= B activation rows are real: the others re-read row Bn - 1 and are not
// stored. kspan: the K range of one split (a multiple of kGqWaveK); with one split the
// block writes y (TY), otherwise its partial sums.
template <bool SYM, int G, int B, int LN, typename TY>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4))) void gptq_gemv_kernel(const uint32_t* __restrict__ qweight,
                                                        const uint16_t* __restrict__ scale_bits,
                                                        const uint32_t* __restrict__ qzeros, int N, int K,
                                                        int kspan, const uint16_t* __restrict__ x, int64_t ldx,
                                                        int Bn, float* __restrict__ part, TY* __restrict__ y,
                                                        int64_t ldy) {
  static_assert(kGqWaveK % G == 0, "a wavefront covers whole groups");
  constexpr int WN = 64 * LN;                           // columns per wavefront
  __shared__ float red[4][B][WN];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int n0 = blockIdx.x * WN + lane * LN;
  const int nc = min(n0, N - LN);                       // N % 8 == 0: lanes past N read a valid place
  const int ks = blockIdx.y * kspan, ke = min(K, ks + kspan);
  const int per = ((ke - ks + kGqWaveK - 1) / kGqWaveK + 3) / 4;   // steps per band
  const int kbeg = ks + wave * per * kGqWaveK, kend = min(ke, kbeg + per * kGqWaveK);
  float acc[B][LN];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int j = 0; j < LN; ++j) acc[b][j] = 0.0f;
  // wave-uniform steps; K % G == 0, so every step holds whole groups, and all but the
  // last of a band cover kGqWaveK k
  for (int kw = kbeg; kw < kend; kw += kGqWaveK) {
    const int nr = min(kGqWaveK, K - kw) / 8;           // qweight rows of this wavefront
    // batches of more than one row keep the per-row branches: without them the scalar
    // loads of later rows' activations are merged and hoisted past the registers there are
    if (B == 1 && nr == kGqWaveK / 8)
      gq_step<SYM, G, B, LN, true>(qweight, scale_bits, qzeros, N, K, x, ldx, Bn, nc, lane, kw, nr, acc);
    else
      gq_step<SYM, G, B, LN, false>(qweight, scale_bits, qzeros, N, K, x, ldx, Bn, nc, lane, kw, nr, acc);
  }
  // the four bands, added in k order
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int j = 0; j < LN; ++j) red[wave][b][lane * LN + j] = acc[b][j];
  __syncthreads();
  for (int e = t; e < B * WN; e += 256) {
    const int b = e / WN, i = e % WN, n = blockIdx.x * WN + i;
    if (n < N && b < Bn) {
      const float v = ((red[0][b][i] + red[1][b][i]) + red[2][b][i]) + red[3][b][i];
      if (gridDim.y == 1) store_y(y + (int64_t)b * ldy + n, v);
      else part[((int64_t)blockIdx.y * Bn + b) * N + n] = v;
    }
  }
}

// ------------------------------------------------------------------ GPTQ act-order
// Act-order GPTQ (channel k in group g_idx[k], gptq_act.hip): the per-group factoring
// above does not apply, so each weight is formed: w = (c - z) s, exact in float32 as one
// fma (5-bit code difference, fp16 scale). A block covers 64 columns, one qweight word
// per lane, and its four wavefronts take 128-k steps of its K range in turn; for every
// k the group g_idx[k] is the same across the wavefront and picks each column's scale and
// zero point from LDS, which holds every group's for the block's columns. Products with
// the bf16 activations are exact; sums are float32 in k order per wavefront.
// TAB (up to kActTabGroups groups): LDS holds each (group, column)'s float32 pair
// (s, -z s), both exact, so a weight is one 8-byte LDS read and one fma; otherwise the
// fp16 scale bits and the qzeros words (a fifth of the bytes), widened per weight.
constexpr int kActGvCols = 64;
constexpr int kActTabGroups = 96;   // 48 KB of (s, -z s) pairs per block

template <bool SYM, int B, typename TY, bool TAB>
__global__ __launch_bounds__(256) void gptq_act_gemv_kernel(const uint32_t* __restrict__ qweight,
                                                            const uint16_t* __restrict__ scale_bits,
                                                            const uint32_t* __restrict__ qzeros,
                                                            const int32_t* __restrict__ g_idx, int N, int K, int NG,
                                                            int kspan, const uint16_t* __restrict__ x, int64_t ldx,
                                                            int Bn, float* __restrict__ part, TY* __restrict__ y,
                                                            int64_t ldy) {
  extern __shared__ uint32_t lds[];
  uint16_t* sl = reinterpret_cast<uint16_t*>(lds);             // [NG][64] fp16 scale bits
  uint32_t* zl = lds + NG * (kActGvCols / 2);                    // [NG][8] qzeros words
  float2* tz = reinterpret_cast<float2*>(lds);                   // TAB: [NG][64] (s, -z s)
  __shared__ float red[4][B][kActGvCols];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int n0 = blockIdx.x * kActGvCols;
  const int nc = min(n0 + lane, N - 1);                         // lanes past N read a valid place
  if constexpr (TAB) {
    for (int e = t; e < NG * kActGvCols; e += 256) {
      const int g = e / kActGvCols, c = e - g * kActGvCols, n = n0 + c;
      float sc = 0.0f, z = 8.0f;
      if (n < N) {
        sc = (float)__builtin_bit_cast(_Float16, scale_bits[(int64_t)g * N + n]);
        if constexpr (!SYM) z = (float)((qzeros[(int64_t)g * (N / 8) + n / 8] >> (4 * (n % 8))) & 0xFu);
      }
      tz[e] = float2{sc, -(z * sc)};
    }
  } else {
    for (int e = t; e < NG * kActGvCols; e += 256) {
      const int g = e / kActGvCols, c = e - g * kActGvCols;
      sl[e] = n0 + c < N ? scale_bits[(int64_t)g * N + n0 + c] : (uint16_t)0;
    }
    if constexpr (!SYM) {
      for (int e = t; e < NG * (kActGvCols / 8); e += 256) {
        const int g = e / (kActGvCols / 8), q = e - g * (kActGvCols / 8);
        zl[e] = n0 + 8 * q < N ? qzeros[(int64_t)g * (N / 8) + n0 / 8 + q] : 0u;
      }
    }
  }
  __syncthreads();
  const int kend = min(K, (int)(blockIdx.y + 1) * kspan);
  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.0f;
  for (int kw = blockIdx.y * kspan + wave * 128; kw < kend; kw += 512) {   // wave-uniform
    const int nr = min(128, K - kw) / 8;
    uint32_t wv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (r < nr) wv[r] = ld4_nt(qweight + (int64_t)(kw / 8 + r) * N + nc);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (r >= nr) continue;                                    // wave-uniform
      const int k = kw + 8 * r;
      const U4 ga = ld16(g_idx + k), gb = ld16(g_idx + k + 4);
      const uint32_t g8[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
      float xk[B][8];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const U4 xv = *reinterpret_cast<const U4*>(x + (int64_t)min(b, Bn - 1) * ldx + k);
        xk[b][0] = bf16_lo(xv.x); xk[b][1] = bf16_hi(xv.x); xk[b][2] = bf16_lo(xv.y); xk[b][3] = bf16_hi(xv.y);
        xk[b][4] = bf16_lo(xv.z); xk[b][5] = bf16_hi(xv.z); xk[b][6] = bf16_lo(xv.w); xk[b][7] = bf16_hi(xv.w);
      }
      uint32_t ev = wv[r] & 0x0F0F0F0Fu, od = (wv[r] >> 4) & 0x0F0F0F0Fu;
      asm volatile("" : "+v"(ev), "+v"(od));   // codes convert from their bytes (v_cvt_f32_ubyte)
      const float cf[8] = {(float)(ev & 0xFFu), (float)(od & 0xFFu), (float)((ev >> 8) & 0xFFu),
                           (float)((od >> 8) & 0xFFu), (float)((ev >> 16) & 0xFFu), (float)((od >> 16) & 0xFFu),
                           (float)(ev >> 24), (float)(od >> 24)};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t g = g8[i] < (uint32_t)NG ? g8[i] : (uint32_t)(NG - 1);   // clamped into range
        float w;
        if constexpr (TAB) {
          const float2 sz = tz[g * kActGvCols + lane];
          w = __builtin_fmaf(cf[i], sz.x, sz.y);
        } else {
          const float sc = (float)__builtin_bit_cast(_Float16, sl[g * kActGvCols + lane]);
          float z = 8.0f;
          if constexpr (!SYM) z = (float)((zl[g * (kActGvCols / 8) + lane / 8] >> (4 * (lane % 8))) & 0xFu);
          w = __builtin_fmaf(cf[i], sc, -(z * sc));
        }
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = __builtin_fmaf(w, xk[b][i], acc[b]);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < B; ++b) red[wave][b][lane] = acc[b];
  __syncthreads();
  for (int e = t; e < B * kActGvCols; e += 256) {
    const int b = e / kActGvCols, i = e - b * kActGvCols, n = n0 + i;
    if (n < N && b < Bn) {
      const float v = ((red[0][b][i] + red[1][b][i]) + red[2][b][i]) + red[3][b][i];
      if (gridDim.y == 1) store_y(y + (int64_t)b * ldy + n, v);
      else part[((int64_t)blockIdx.y * Bn + b) * N + n] = v;
    }
  }
}

// Act-order GPTQ for batches of three to eight rows: two columns per lane (a block covers
// 128), so one 16-byte LDS read gives both columns' (s, -z s) for a group and each
// activation value feeds two columns; same products and the same k-order sums per
// column as the kernel above. Measured on the 131072 x 2048 head: 14% less time at four
// rows, about 20% at eight, and more at one and two rows (half as many blocks).
constexpr int kAct2Cols = 128;
constexpr int kAct2TabGroups = 48;  // 48 KB of (s, -z s) pairs per block
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <bool SYM, int B, typename TY>
__global__ __launch_bounds__(256) void gptq_act_gemv2_kernel(const uint32_t* __restrict__ qweight,
                                                             const uint16_t* __restrict__ scale_bits,
                                                             const uint32_t* __restrict__ qzeros,
                                                             const int32_t* __restrict__ g_idx, int N, int K, int NG,
                                                             int kspan, const uint16_t* __restrict__ x, int64_t ldx,
                                                             int Bn, float* __restrict__ part, TY* __restrict__ y,
                                                             int64_t ldy) {
  extern __shared__ uint32_t lds[];
  float2* tz = reinterpret_cast<float2*>(lds);                   // [NG][128] (s, -z s)
  const float4* tz4 = reinterpret_cast<const float4*>(lds);      // [NG][64] column pairs
  __shared__ float red[4][B][kAct2Cols];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int n0 = blockIdx.x * kAct2Cols;
  const int nc = min(n0 + 2 * lane, N - 2);                     // N % 8 == 0: lanes past N read a valid place
  for (int e = t; e < NG * kAct2Cols; e += 256) {
    const int g = e / kAct2Cols, c = e - g * kAct2Cols, n = n0 + c;
    float sc = 0.0f, z = 8.0f;
    if (n < N) {
      sc = (float)__builtin_bit_cast(_Float16, scale_bits[(int64_t)g * N + n]);
      if constexpr (!SYM) z = (float)((qzeros[(int64_t)g * (N / 8) + n / 8] >> (4 * (n % 8))) & 0xFu);
    }
    tz[e] = float2{sc, -(z * sc)};
  }
  __syncthreads();
  const int kend = min(K, (int)(blockIdx.y + 1) * kspan);
  float acc[B][2];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b][0] = acc[b][1] = 0.0f;
  for (int kw = blockIdx.y * kspan + wave * 128; kw < kend; kw += 512) {   // wave-uniform
    const int nr = min(128, K - kw) / 8;
    u32x2_t wv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (r < nr)
        wv[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(qweight + (int64_t)(kw / 8 + r) * N + nc));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (r >= nr) continue;                                    // wave-uniform
      const int k = kw + 8 * r;
      const U4 ga = ld16(g_idx + k), gb = ld16(g_idx + k + 4);
      const uint32_t g8[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
      float xk[B][8];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const U4 xv = *reinterpret_cast<const U4*>(x + (int64_t)min(b, Bn - 1) * ldx + k);
        xk[b][0] = bf16_lo(xv.x); xk[b][1] = bf16_hi(xv.x); xk[b][2] = bf16_lo(xv.y); xk[b][3] = bf16_hi(xv.y);
        xk[b][4] = bf16_lo(xv.z); xk[b][5] = bf16_hi(xv.z); xk[b][6] = bf16_lo(xv.w); xk[b][7] = bf16_hi(xv.w);
      }
      float cf[2][8];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint32_t ev = wv[r][j] & 0x0F0F0F0Fu, od = (wv[r][j] >> 4) & 0x0F0F0F0Fu;
        asm volatile("" : "+v"(ev), "+v"(od));   // codes convert from their bytes (v_cvt_f32_ubyte)
        cf[j][0] = (float)(ev & 0xFFu); cf[j][1] = (float)(od & 0xFFu); cf[j][2] = (float)((ev >> 8) & 0xFFu);
        cf[j][3] = (float)((od >> 8) & 0xFFu); cf[j][4] = (float)((ev >> 16) & 0xFFu);
        cf[j][5] = (float)((od >> 16) & 0xFFu); cf[j][6] = (float)(ev >> 24); cf[j][7] = (float)(od >> 24);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t g = g8[i] < (uint32_t)NG ? g8[i] : (uint32_t)(NG - 1);   // clamped into range
        const float4 sz = tz4[g * (kAct2Cols / 2) + lane];
        const float w0 = __builtin_fmaf(cf[0][i], sz.x, sz.y), w1 = __builtin_fmaf(cf[1][i], sz.z, sz.w);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          acc[b][0] = __builtin_fmaf(w0, xk[b][i], acc[b][0]);
          acc[b][1] = __builtin_fmaf(w1, xk[b][i], acc[b][1]);
        }
      }
    }
  }
#pragma unroll
  for (int b = 0; b < B; ++b) {
    red[wave][b][2 * lane] = acc[b][0];
    red[wave][b][2 * lane + 1] = acc[b][1];
  }
  __syncthreads();
  for (int e = t; e < B * kAct2Cols; e += 256) {
    const int b = e / kAct2Cols, i = e - b * kAct2Cols, n = n0 + i;
    if (n < N && b < Bn) {
      const float v = ((red[0][b][i] + red[1][b][i]) + red[2][b][i]) + red[3][b][i];
      if (gridDim.y == 1) store_y(y + (int64_t)b * ldy + n, v);
      else part[((int64_t)blockIdx.y * Bn + b) * N + n] = v;
    }
  }
}

// y[b, n] = sum over the K splits of part[s][b][n], in order.
template <typename TY>
__global__ __launch_bounds__(256) void gemv_finalize_kernel(const float* __restrict__ part, int S, int B, int N,
                                                            TY* __restrict__ y, int64_t ldy) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)B * N) return;
  const int b = (int)(e / N), n = (int)(e % N);
  float v = 0.0f;
  for (int s = 0; s < S; ++s) v += part[((int64_t)s * B + b) * N + n];
  store_y(y + (int64_t)b * ldy + n, v);
}

// ------------------------------------------------------------------ MXFP4
template <int B> struct MxRows { static constexpr int R = B <= 2 ? 8 : (B <= 4 ? 4 : 2); };

template <int B>
__device__ __forceinline__ void load_x_block(const uint16_t* __restrict__ x, int64_t ldx, int blk, uint32_t (&xa)[B][16]) {
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const U4* xp = reinterpret_cast<const U4*>(x + (int64_t)b * ldx + 32 * blk);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const U4 v = xp[q];
      xa[b][4 * q] = v.x; xa[b][4 * q + 1] = v.y; xa[b][4 * q + 2] = v.z; xa[b][4 * q + 3] = v.w;
    }
  }
}

// Sum over the 32-blocks lane, lane + 64, ... of row n that have a scale byte of 255, of
// the activations xr times the page's weights there (+-E2M1 * 2^128: inf, or NaN for a
// zero code), in float32. Out of line: the rare path keeps its registers out of the
// main loop.
__device__ __attribute__((noinline)) float mx_nan_lane_sum(const uint8_t* __restrict__ packed,
                                                           const uint8_t* __restrict__ e8m0, int K, int n,
                                                           const uint16_t* __restrict__ xr, int lane) {
  const int nblk = K / 32;
  const uint8_t* crow = packed + (int64_t)n * (K / 2);
  float sum = 0.0f;
  for (int blk = lane; blk < nblk; blk += 64) {
    if (e8m0[(int64_t)n * nblk + blk] != 255u) continue;
    for (int k = 32 * blk; k < 32 * blk + 32; ++k)
      sum += bf16_to_f32(xr[k]) * mx_value_nan_scale((crow[k >> 1] >> (4 * (k & 1))) & 0xFu);
  }
  return sum;
}

template <int B, typename TY>
__global__ __launch_bounds__(256) void mxfp4_gemv_kernel(const uint8_t* __restrict__ packed,
                                                         const uint8_t* __restrict__ e8m0, int N, int K,
                                                         const uint16_t* __restrict__ x, int64_t ldx,
                                                         TY* __restrict__ y, int64_t ldy) {
  constexpr int R = MxRows<B>::R;
  const int lane = threadIdx.x & 63;
  const int nblk = K / 32;                            // blocks per row
  const int steps = (nblk + 63) / 64;                 // blocks per lane
  const int waves = gridDim.x * 4;
  const int wave = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const float one = mx_scale_operand(127u);
  uint32_t xa[B][16];                                 // activation pairs of the lane's block
  if (steps == 1) load_x_block<B>(x, ldx, min(lane, nblk - 1), xa);
  for (int row0 = wave * R; row0 < N; row0 += waves * R) {     // wave-uniform
    float acc[R][B];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int b = 0; b < B; ++b) acc[i][b] = 0.0f;
    uint32_t nanm = 0;                                  // bit i: this lane has a block of row i with scale byte 255
    for (int st = 0; st < steps; ++st) {
      const int blk = st * 64 + lane;
      const bool ok = blk < nblk;
      const int bc = ok ? blk : nblk - 1;
      if (steps != 1) load_x_block<B>(x, ldx, bc, xa);
      U4 pw[R];
      uint32_t ev[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int n = min(row0 + i, N - 1);
        pw[i] = ld16_nt(packed + (int64_t)n * (K / 2) + 16 * bc);
        ev[i] = e8m0[(int64_t)n * nblk + bc];
      }
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const uint32_t w[4] = {pw[i].x, pw[i].y, pw[i].z, pw[i].w};
        float d[B];
#pragma unroll
        for (int b = 0; b < B; ++b) d[b] = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          gv_bf16x2_t v[4];
          v[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], one, 0);
          v[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], one, 1);
          v[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], one, 2);
          v[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], one, 3);
#pragma unroll
          for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int b = 0; b < B; ++b)
              d[b] = __builtin_amdgcn_fdot2_f32_bf16(v[p], __builtin_bit_cast(gv_bf16x2_t, xa[b][4 * q + p]), d[b],
                                                     false);
        }
        const int ex = (int)ev[i] - 127;
        nanm |= (uint32_t)(ok && ev[i] == 255u) << i;
#pragma unroll
        for (int b = 0; b < B; ++b) acc[i][b] += ok ? ldexpf(d[b], ex) : 0.0f;
      }
    }
    // Blocks with a scale byte of 255 (no E8M0 value): the page's weights +-E2M1 * 2^128
    // are inf or NaN (NaN for a zero code), so such a lane's sum for that row becomes the
    // float32 sum over its 255 blocks alone, which adding the finite rest cannot change.
    if (__any(nanm != 0u)) {                                    // wave-uniform, rare
#pragma unroll
      for (int i = 0; i < R; ++i) {
        if (!((nanm >> i) & 1u)) continue;
        const int n = min(row0 + i, N - 1);
#pragma unroll
        for (int b = 0; b < B; ++b) acc[i][b] = mx_nan_lane_sum(packed, e8m0, K, n, x + (int64_t)b * ldx, lane);
      }
    }
    // value i B + b (row i, activation row b), padded with zeros to VP
    constexpr int V = R * B, VP = V <= 8 ? 8 : 16;
    float v[VP];
#pragma unroll
    for (int e = 0; e < VP; ++e) v[e] = e < V ? acc[e / B][e % B] : 0.0f;
    const float sum = gv_transposed_sum<VP>(v, lane);
    const int e = lane & (VP - 1), i = e / B, b = e - i * B;
    if (lane < V && row0 + i < N) store_y(y + (int64_t)b * ldy + row0 + i, sum);
  }
}

// ------------------------------------------------------------------ MXFP4, batches on the matrix cores
// Five to eight activation rows: v_mfma_f32_16x16x32_bf16 with the weights as A (16 rows
// x 32 k) and the activations as B (32 k x 16 columns, one per activation row; columns
// past the batch repeat the last row and are not stored). A wavefront takes tiles of 16
// weight rows. Per 128 k, lane (j = l % 16, q = l / 16) loads the 16 bytes of 32-block
// k0 + 32q of row j; their scaled FP4 conversion gives the exact bf16 weights of four A
// fragments, slot q of MFMA s holding k0 + 32q + 8s .. +7, and the B fragment of that slot
// is x[j][k0 + 32q + 8s .. +7] (the same relabelling of k on both sides). Lane (j, q)
// ends with weight rows 4q .. 4q + 3 for activation row j. Products are exact; the sums
// are the matrix cores' float32 sums.
// K splits of at most mxm_chunk(B) k (blockIdx.y) keep a block's activations in LDS,
// staged once; with more than one split each writes float32 partials, added in split
// order afterwards. The blocks are persistent, and a wavefront's loads run one batch
// (kMxmNS steps of 128 k) ahead of its products, across tile boundaries, from two
// register buffers.
constexpr int kMxmNS = 8;
constexpr int kMxmLds = 8 * 2056 * 2;               // activation bytes staged per block: 8 rows of 2048 k
// From 5 activation rows (measured on the 131072 x 2048 lm_head: B = 8 37 us against 45
// for the GEMM tiles and 75 for the 32-block GEMV kernel; B <= 4 the GEMV kernel is as
// fast or faster: each of its loads reads 1 KB of one row, the matrix-core order 64 bytes
// of each of 16 rows).
constexpr int kMxmMinRows = 5;

// K per split for B activation rows: B (kc + 8) bf16 within kMxmLds bytes, a multiple
// of the 1024 k of a batch.
__host__ __device__ constexpr int mxm_chunk(int B) { return (kMxmLds / (2 * B) - 8) / 1024 * 1024; }
int mxfp4_gemv_splits(int64_t K, int B) {
  if (B < kMxmMinRows) return 1;
  const int64_t kc = mxm_chunk(B);
  return (int)((K + kc - 1) / kc);
}

typedef __bf16 gv_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float gv_f32x4_t __attribute__((ext_vector_type(4)));

struct MxmBuf {
  U4 w[kMxmNS];
  uint32_t e[kMxmNS];   // AL: the batch's 32 scale bytes of the row (step i's block q in byte q of e[i]); else step i's byte
};

// The loads of one batch: steps k0 + 128 i. AL (K % 1024 == 0: every batch lies inside
// its split, and rows of scale bytes are 16-byte aligned): the row's 32 scale bytes of
// the batch in two 16-byte loads; otherwise one byte per step, and slots past the split
// end re-read its last block. live == false points every lane at the row's first bytes
// (a prefetch past the wavefront's last tile), so the instruction count never depends on
// data.
template <bool AL>
__device__ __forceinline__ void mxm_load(MxmBuf& bf, const uint8_t* __restrict__ wr, const uint8_t* __restrict__ er,
                                         int k0, int kend, int q, bool live) {
#pragma unroll
  for (int i = 0; i < kMxmNS; ++i) {
    const int kk = !live ? 0 : AL ? k0 + 128 * i + 32 * q : min(k0 + 128 * i + 32 * q, kend - 32);
    bf.w[i] = ld16_nt(wr + kk / 2);
    if constexpr (!AL) bf.e[i] = er[kk / 32];
  }
  if constexpr (AL) {
    const uint8_t* ep = er + (live ? k0 / 32 : 0);
    const U4 lo = ld16(ep), hi = ld16(ep + 16);
    bf.e[0] = lo.x; bf.e[1] = lo.y; bf.e[2] = lo.z; bf.e[3] = lo.w;
    bf.e[4] = hi.x; bf.e[5] = hi.y; bf.e[6] = hi.z; bf.e[7] = hi.w;
  }
}

// The products of one batch; xb: this lane's activation row in LDS, from the split start.
// FULL: the whole batch lies inside the split.
template <bool AL, bool FULL>
__device__ __forceinline__ void mxm_mma(const MxmBuf& bf, const uint16_t* xb, int k0, int ks, int kend, int q,
                                        gv_f32x4_t& acc, uint32_t& nan) {
  static_assert(kMxmNS == 8, "a batch's scale bytes are two 16-byte loads");
#pragma unroll
  for (int i = 0; i < kMxmNS; ++i) {
    const int k = k0 + 128 * i;
    if (FULL || k < kend) {                                     // wave-uniform
      const int kl = k + 32 * q;                                // this lane's 32-block
      const bool ok = FULL || kl < kend;                        // inside the split
      const uint32_t e8 = AL ? (bf.e[i] >> (8 * q)) & 0xFFu : bf.e[i];
      const float scl = mx_scale_operand(e8);
      nan |= (uint32_t)(ok && e8 == 255u);
      U4 b[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        b[s] = *reinterpret_cast<const U4*>(xb + (ok ? (kl - ks) + 8 * s : 0));   // inside the staged row
        if (!ok) b[s] = U4{0u, 0u, 0u, 0u};
      }
      const U4 w = bf.w[i];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t wd = s == 0 ? w.x : s == 1 ? w.y : s == 2 ? w.z : w.w;
        U4 a{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 0)),
             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 1)),
             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 2)),
             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 3))};
        if (!ok) a = U4{0u, 0u, 0u, 0u};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gv_bf16x8_t, a),
                                                      __builtin_bit_cast(gv_bf16x8_t, b[s]), acc, 0, 0, 0);
      }
    }
  }
}

// Rows of a tile with a scale byte of 255 in the split [ks, kend): lane (j, q)'s outputs
// 4q + r of those rows become the float32 sum of x[j] times the page's inf or NaN weights
// over the split's such blocks. Out of line: the common path keeps its load bookkeeping.
__device__ __attribute__((noinline)) gv_f32x4_t mxm_nan_rows(const uint8_t* __restrict__ packed,
                                                             const uint8_t* __restrict__ e8m0, int N, int K,
                                                             const uint16_t* __restrict__ x, int64_t ldx, int ks,
                                                             int kend, int n0, int j, int q, bool bcol, uint32_t rows,
                                                             gv_f32x4_t acc) {
  const int64_t rowb = K / 2, rowe = K / 32;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (!((rows >> (4 * q + r)) & 1u) || !bcol) continue;
    const int n = min(n0 + 4 * q + r, N - 1);
    const uint8_t* crow = packed + n * rowb;
    const uint8_t* erow = e8m0 + n * rowe;
    const uint16_t* xr = x + (int64_t)j * ldx;
    float sum = 0.f;
    for (int blk = ks / 32; blk < kend / 32; ++blk) {
      if (erow[blk] != 255u) continue;
      for (int k = 32 * blk; k < 32 * blk + 32; ++k)
        sum += bf16_to_f32(xr[k]) * mx_value_nan_scale((crow[k >> 1] >> (4 * (k & 1))) & 0xFu);
    }
    acc[r] = sum;
  }
  return acc;
}

template <typename TY, bool AL>
__global__ __launch_bounds__(256) void mxfp4_gemv_mfma_kernel(const uint8_t* __restrict__ packed,
                                                              const uint8_t* __restrict__ e8m0, int N, int K,
                                                              const uint16_t* __restrict__ x, int64_t ldx, int Bn,
                                                              TY* __restrict__ y, int64_t ldy,
                                                              float* __restrict__ part) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // [Bn][kc + 8]
  const int t = threadIdx.x, lane = t & 63, j = lane & 15, q = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t rowb = K / 2, rowe = K / 32;
  const int kc = mxm_chunk(Bn), xp = kc + 8;
  const int ks = (int)blockIdx.y * kc, kend = min(K, ks + kc);   // this split: [ks, kend), a multiple of 32
  const int nb = (kend - ks + 128 * kMxmNS - 1) / (128 * kMxmNS);   // batches per tile
  const int nbt = (N + 63) / 64;                                // 64-row block tiles
  const uint16_t* xb = xs + min(j, Bn - 1) * xp;                // rows past the batch repeat the last
  const bool bcol = j < Bn;
  auto rows_of = [&](int bt, const uint8_t*& wr, const uint8_t*& er) {
    const int nl = min((bt * 4 + wave) * 16 + j, N - 1);        // rows past N read a valid row, not stored
    wr = packed + nl * rowb;
    er = e8m0 + nl * rowe;
  };
  // finish a tile: rows with a scale byte of 255 (no E8M0 value; the page's weights
  // +-E2M1 * 2^128 are inf or NaN) get the float32 sum over the split's such blocks alone,
  // which adding the finite rest cannot change; then the rows are stored
  auto finish = [&](int bt, gv_f32x4_t& acc, uint32_t& nan) {
    const int n0 = (bt * 4 + wave) * 16;
    const uint64_t m = __ballot(nan != 0u);
    const uint32_t rows = (uint32_t)((m | (m >> 16) | (m >> 32) | (m >> 48)) & 0xFFFFu);
    if (rows != 0u) acc = mxm_nan_rows(packed, e8m0, N, K, x, ldx, ks, kend, n0, j, q, bcol, rows, acc);   // rare
    if (bcol) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n0 + 4 * q + r;
        if (n >= N) continue;
        if (gridDim.y == 1) store_y(y + (int64_t)j * ldy + n, acc[r]);
        else part[((int64_t)blockIdx.y * Bn + j) * N + n] = acc[r];
      }
    }
    acc = gv_f32x4_t{0.f, 0.f, 0.f, 0.f};
    nan = 0u;
  };
  int bt = blockIdx.x, h = 0;                                   // block-uniform, below nbt (the grid is capped)
  gv_f32x4_t acc = gv_f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint32_t nan = 0u;
  const uint8_t *wr, *er;
  rows_of(bt, wr, er);
  MxmBuf b0, b1;
  mxm_load<AL>(b0, wr, er, ks, kend, q, true);                  // the weight stream starts before the staging
  asm volatile("" ::: "memory");
  // the split's activations, staged once (rows in LDS padded by 16 bytes: no bank conflicts)
  stage_rows(xs, xp, x, ldx, Bn, ks, kend);
  __syncthreads();
  // two items per trip, one per buffer: load the next item, then multiply the current
  for (;;) {
    int bt2 = bt, h2 = h + 1;
    if (h2 == nb) { h2 = 0; bt2 += gridDim.x; }
    bool more = bt2 < nbt;
    const uint8_t *wr2 = wr, *er2 = er;
    if (bt2 != bt && more) rows_of(bt2, wr2, er2);
    mxm_load<AL>(b1, wr2, er2, ks + h2 * 128 * kMxmNS, kend, q, more);
    asm volatile("" ::: "memory");       // keep the loads here, ahead of the products
    __builtin_amdgcn_sched_barrier(0);
    if (AL || ks + (h + 1) * 128 * kMxmNS <= kend) mxm_mma<AL, true>(b0, xb, ks + h * 128 * kMxmNS, ks, kend, q, acc, nan);
    else mxm_mma<AL, false>(b0, xb, ks + h * 128 * kMxmNS, ks, kend, q, acc, nan);
    if (h == nb - 1) finish(bt, acc, nan);
    if (!more) break;
    bt = bt2; h = h2; wr = wr2; er = er2;

    bt2 = bt; h2 = h + 1;
    if (h2 == nb) { h2 = 0; bt2 += gridDim.x; }
    more = bt2 < nbt;
    wr2 = wr; er2 = er;
    if (bt2 != bt && more) rows_of(bt2, wr2, er2);
    mxm_load<AL>(b0, wr2, er2, ks + h2 * 128 * kMxmNS, kend, q, more);
    asm volatile("" ::: "memory");       // keep the loads here, ahead of the products
    __builtin_amdgcn_sched_barrier(0);
    if (AL || ks + (h + 1) * 128 * kMxmNS <= kend) mxm_mma<AL, true>(b1, xb, ks + h * 128 * kMxmNS, ks, kend, q, acc, nan);
    else mxm_mma<AL, false>(b1, xb, ks + h * 128 * kMxmNS, ks, kend, q, acc, nan);
    if (h == nb - 1) finish(bt, acc, nan);
    if (!more) break;
    bt = bt2; h = h2; wr = wr2; er = er2;
  }
}

// ------------------------------------------------------------------ launchers
// Outputs per lane: 4 (one 16-byte load per qweight row). One and two measured the same
// for one activation row and slower for four: the kernel is VALU-bound there.
constexpr int kGqLaneN = 4;
// K splits: none when the column chunks alone give kGqMinBlocks blocks (a second pass
// costs more than it gains there); otherwise enough for about kGqSplitBlocks blocks, at
// most one per four wavefront steps of K. Measured on MI355X: contiguous K bands per
// wavefront read faster than wavefronts on interleaved 128-k steps, and one 1 KB column
// chunk per block faster than two or four neighbouring chunks.
constexpr int kGqMinBlocks = 512, kGqSplitBlocks = 1024;
constexpr int kGqBandK = 4 * kGqWaveK;                   // one step of each of a block's bands
int gptq_gemv_splits(int64_t N, int64_t K) {
  const int64_t wn = 64 * kGqLaneN;
  const int64_t tiles = (N + wn - 1) / wn, kb = (K + kGqBandK - 1) / kGqBandK;
  if (tiles >= kGqMinBlocks) return 1;
  const int64_t want = (kGqSplitBlocks + tiles - 1) / tiles;
  const int64_t per = (kb + (want > kb ? kb : want) - 1) / (want > kb ? kb : want);   // units per split
  return (int)((kb + per - 1) / per);                   // every split holds some of K
}

template <bool SYM, int G, int B, int LN, typename TY>
static void gptq_gemv_ln(int Bn, const void* qw, const void* sc, const void* qz, int64_t N, int64_t K, const void* x,
                         int64_t ldx, float* part, void* y, int64_t ldy, hipStream_t st) {
  const int S = gptq_gemv_splits(N, K);
  const int64_t kb = (K + kGqBandK - 1) / kGqBandK;
  const int kspan = (int)((kb + S - 1) / S) * kGqBandK;
  const dim3 grid((unsigned)((N + 64 * LN - 1) / (64 * LN)), (unsigned)S);
  hipLaunchKernelGGL((gptq_gemv_kernel<SYM, G, B, LN, TY>), grid, dim3(256), 0, st, (const uint32_t*)qw,
                     (const uint16_t*)sc, (const uint32_t*)qz, (int)N, (int)K, kspan, (const uint16_t*)x, ldx, Bn,
                     part, (TY*)y, ldy);
}
template <bool SYM, int G, int B, typename TY>
static void gptq_gemv_b(int Bn, const void* qw, const void* sc, const void* qz, int64_t N, int64_t K, const void* x,
                        int64_t ldx, float* part, void* y, int64_t ldy, hipStream_t st) {
  gptq_gemv_ln<SYM, G, B, kGqLaneN, TY>(Bn, qw, sc, qz, N, K, x, ldx, part, y, ldy, st);
}

template <bool SYM, int G, typename TY>
static void gptq_gemv_g(int B, const void* qw, const void* sc, const void* qz, int64_t N, int64_t K, const void* x,
                        int64_t ldx, float* part, void* y, int64_t ldy, hipStream_t st) {
  if (B == 1) gptq_gemv_b<SYM, G, 1, TY>(B, qw, sc, qz, N, K, x, ldx, part, y, ldy, st);
  else if (B == 2) gptq_gemv_b<SYM, G, 2, TY>(B, qw, sc, qz, N, K, x, ldx, part, y, ldy, st);
  else if (B <= 4) gptq_gemv_b<SYM, G, 4, TY>(B, qw, sc, qz, N, K, x, ldx, part, y, ldy, st);
  else gptq_gemv_b<SYM, G, 8, TY>(B, qw, sc, qz, N, K, x, ldx, part, y, ldy, st);
}

template <bool SYM, typename TY>
static void gptq_gemv_s(int group, int B, const void* qw, const void* sc, const void* qz, int64_t N, int64_t K,
                        const void* x, int64_t ldx, float* part, void* y, int64_t ldy, hipStream_t st) {
  if (group == 32) gptq_gemv_g<SYM, 32, TY>(B, qw, sc, qz, N, K, x, ldx, part, y, ldy, st);
  else if (group == 64) gptq_gemv_g<SYM, 64, TY>(B, qw, sc, qz, N, K, x, ldx, part, y, ldy, st);
  else gptq_gemv_g<SYM, 128, TY>(B, qw, sc, qz, N, K, x, ldx, part, y, ldy, st);
}

void launch_gptq_gemv(bool sym, int group, int B, const void* qweight, const void* scales, const void* qzeros,
                      int64_t N, int64_t K, const void* x, int64_t ldx, void* y, int32_t y_dtype, int64_t ldy,
                      float* part, hipStream_t st) {
  if (y_dtype == kBF16) {
    if (sym) gptq_gemv_s<true, uint16_t>(group, B, qweight, scales, qzeros, N, K, x, ldx, part, y, ldy, st);
    else gptq_gemv_s<false, uint16_t>(group, B, qweight, scales, qzeros, N, K, x, ldx, part, y, ldy, st);
  } else {
    if (sym) gptq_gemv_s<true, float>(group, B, qweight, scales, qzeros, N, K, x, ldx, part, y, ldy, st);
    else gptq_gemv_s<false, float>(group, B, qweight, scales, qzeros, N, K, x, ldx, part, y, ldy, st);
  }
  const int S = gptq_gemv_splits(N, K);
  if (S > 1) launch_gemv_finalize(part, S, B, N, y, y_dtype, ldy, st);
}

constexpr int kActMinBlocks = 512;
int gptq_act_gemv_splits(int64_t N, int64_t K) {
  const int64_t tiles = (N + kActGvCols - 1) / kActGvCols, kb = (K + 511) / 512;
  const int64_t want = (kActMinBlocks + tiles - 1) / tiles;
  return (int)(want < 1 ? 1 : (want > kb ? kb : want));
}

template <bool SYM, int B, typename TY>
static void act_gemv_b(int Bn, int group, const void* qw, const void* sc, const void* qz, const int32_t* g_idx,
                       int64_t N, int64_t K, const void* x, int64_t ldx, float* part, void* y, int64_t ldy,
                       hipStream_t st) {
  const int S = gptq_act_gemv_splits(N, K), NG = (int)(K / group);
  const int64_t kb = (K + 511) / 512;
  const int kspan = (int)((kb + S - 1) / S) * 512;
  const dim3 grid((unsigned)((N + kActGvCols - 1) / kActGvCols), (unsigned)S);
  if (B >= 4 && NG <= kAct2TabGroups && (reinterpret_cast<uintptr_t>(qw) & 7) == 0) {
    // the same K splits as the one-column kernel (the workspace is sized by them)
    const dim3 grid2((unsigned)((N + kAct2Cols - 1) / kAct2Cols), (unsigned)S);
    const size_t lds = (size_t)NG * kAct2Cols * sizeof(float2);
    hipLaunchKernelGGL((gptq_act_gemv2_kernel<SYM, B, TY>), grid2, dim3(256), lds, st, (const uint32_t*)qw,
                       (const uint16_t*)sc, (const uint32_t*)qz, g_idx, (int)N, (int)K, NG, kspan,
                       (const uint16_t*)x, ldx, Bn, part, (TY*)y, ldy);
  } else if (NG <= kActTabGroups) {
    const size_t lds = (size_t)NG * kActGvCols * sizeof(float2);
    hipLaunchKernelGGL((gptq_act_gemv_kernel<SYM, B, TY, true>), grid, dim3(256), lds, st, (const uint32_t*)qw,
                       (const uint16_t*)sc, (const uint32_t*)qz, g_idx, (int)N, (int)K, NG, kspan,
                       (const uint16_t*)x, ldx, Bn, part, (TY*)y, ldy);
  } else {
    const size_t lds = (size_t)NG * (kActGvCols * 2 + (SYM ? 0 : (kActGvCols / 8) * 4));
    hipLaunchKernelGGL((gptq_act_gemv_kernel<SYM, B, TY, false>), grid, dim3(256), lds, st, (const uint32_t*)qw,
                       (const uint16_t*)sc, (const uint32_t*)qz, g_idx, (int)N, (int)K, NG, kspan,
                       (const uint16_t*)x, ldx, Bn, part, (TY*)y, ldy);
  }
}
template <bool SYM, typename TY>
static void act_gemv_s(int B, int group, const void* qw, const void* sc, const void* qz, const int32_t* g_idx,
                       int64_t N, int64_t K, const void* x, int64_t ldx, float* part, void* y, int64_t ldy,
                       hipStream_t st) {
  if (B == 1) act_gemv_b<SYM, 1, TY>(B, group, qw, sc, qz, g_idx, N, K, x, ldx, part, y, ldy, st);
  else if (B == 2) act_gemv_b<SYM, 2, TY>(B, group, qw, sc, qz, g_idx, N, K, x, ldx, part, y, ldy, st);
  else if (B <= 4) act_gemv_b<SYM, 4, TY>(B, group, qw, sc, qz, g_idx, N, K, x, ldx, part, y, ldy, st);
  else act_gemv_b<SYM, 8, TY>(B, group, qw, sc, qz, g_idx, N, K, x, ldx, part, y, ldy, st);
}

void launch_gptq_act_gemv(bool sym, int group, int B, const void* qweight, const void* scales, const void* qzeros,
                          const int32_t* g_idx, int64_t N, int64_t K, const void* x, int64_t ldx, void* y,
                          int32_t y_dtype, int64_t ldy, float* part, hipStream_t st) {
  if (y_dtype == kBF16) {
    if (sym) act_gemv_s<true, uint16_t>(B, group, qweight, scales, qzeros, g_idx, N, K, x, ldx, part, y, ldy, st);
    else act_gemv_s<false, uint16_t>(B, group, qweight, scales, qzeros, g_idx, N, K, x, ldx, part, y, ldy, st);
  } else {
    if (sym) act_gemv_s<true, float>(B, group, qweight, scales, qzeros, g_idx, N, K, x, ldx, part, y, ldy, st);
    else act_gemv_s<false, float>(B, group, qweight, scales, qzeros, g_idx, N, K, x, ldx, part, y, ldy, st);
  }
  const int S = gptq_act_gemv_splits(N, K);
  if (S > 1) launch_gemv_finalize(part, S, B, N, y, y_dtype, ldy, st);
}

void launch_gemv_finalize(const float* part, int S, int B, int64_t N, void* y, int32_t y_dtype, int64_t ldy,
                          hipStream_t st) {
  const int64_t total = (int64_t)B * N;
  const unsigned fgrid = (unsigned)((total + 255) / 256);
  if (y_dtype == kBF16)
    hipLaunchKernelGGL(gemv_finalize_kernel<uint16_t>, dim3(fgrid), dim3(256), 0, st, part, S, B, (int)N,
                       (uint16_t*)y, ldy);
  else
    hipLaunchKernelGGL(gemv_finalize_kernel<float>, dim3(fgrid), dim3(256), 0, st, part, S, B, (int)N, (float*)y, ldy);
}

template <int B, typename TY>
static void mxfp4_gemv_b(const void* packed, const void* e8m0, int64_t N, int64_t K, const void* x, int64_t ldx,
                         void* y, int64_t ldy, hipStream_t st) {
  const int64_t passes = (N + MxRows<B>::R - 1) / MxRows<B>::R;       // wavefront passes
  const unsigned grid = stream_blocks((uint64_t)passes * 64);          // one wavefront per pass, capped
  hipLaunchKernelGGL((mxfp4_gemv_kernel<B, TY>), dim3(grid), dim3(256), 0, st, (const uint8_t*)packed,
                     (const uint8_t*)e8m0, (int)N, (int)K, (const uint16_t*)x, ldx, (TY*)y, ldy);
}

// Blocks of the matrix-core MXFP4 GEMV that are resident at once (its registers and
// the LDS of B activation rows), times the compute units: the kernel loops over its tiles
// with that many blocks, so none waits for a second round. Cached per device, B, output
// type and variant.
static unsigned mxm_resident_blocks(const void* kern, size_t lds, int B, bool f32, bool al) {
  constexpr int kDev = 64;
  static std::atomic<unsigned> cache[kDev][9][2][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDev) dev = -1;
  if (dev >= 0) {
    const unsigned c = cache[dev][B][f32][al].load(std::memory_order_relaxed);
    if (c) return c;
  }
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) != hipSuccess || cus < 1)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, 256, lds) != hipSuccess || per < 1) per = 1;
  const unsigned r = (unsigned)per * (unsigned)cus;
  if (dev >= 0) cache[dev][B][f32][al].store(r, std::memory_order_relaxed);
  return r;
}

template <typename TY>
static void mxfp4_gemv_t(int B, const void* packed, const void* e8m0, int64_t N, int64_t K, const void* x,
                         int64_t ldx, void* y, int64_t ldy, float* part, hipStream_t st) {
  if (B >= kMxmMinRows) {
    const int S = mxfp4_gemv_splits(K, B);
    const size_t lds = (size_t)B * (mxm_chunk(B) + 8) * sizeof(uint16_t);   // at most kMxmLds
    const int64_t tiles = (N + 63) / 64;
    const bool al = K % 1024 == 0;
    const void* kern = al ? reinterpret_cast<const void*>(&mxfp4_gemv_mfma_kernel<TY, true>)
                          : reinterpret_cast<const void*>(&mxfp4_gemv_mfma_kernel<TY, false>);
    const unsigned res = mxm_resident_blocks(kern, lds, B, sizeof(TY) == 4, al);
    const int64_t per = ((int64_t)res + S - 1) / S;             // blocks per split
    const unsigned gx = (unsigned)(tiles < per ? tiles : per);
    if (al)
      hipLaunchKernelGGL((mxfp4_gemv_mfma_kernel<TY, true>), dim3(gx, (unsigned)S), dim3(256), lds, st,
                         (const uint8_t*)packed, (const uint8_t*)e8m0, (int)N, (int)K, (const uint16_t*)x, ldx, B,
                         (TY*)y, ldy, part);
    else
      hipLaunchKernelGGL((mxfp4_gemv_mfma_kernel<TY, false>), dim3(gx, (unsigned)S), dim3(256), lds, st,
                         (const uint8_t*)packed, (const uint8_t*)e8m0, (int)N, (int)K, (const uint16_t*)x, ldx, B,
                         (TY*)y, ldy, part);
    return;
  }
  switch (B) {
    case 1: mxfp4_gemv_b<1, TY>(packed, e8m0, N, K, x, ldx, y, ldy, st); break;
    case 2: mxfp4_gemv_b<2, TY>(packed, e8m0, N, K, x, ldx, y, ldy, st); break;
    case 3: mxfp4_gemv_b<3, TY>(packed, e8m0, N, K, x, ldx, y, ldy, st); break;
    default: mxfp4_gemv_b<4, TY>(packed, e8m0, N, K, x, ldx, y, ldy, st); break;
  }
}

void launch_mxfp4_gemv(int B, const void* packed, const void* e8m0, int64_t N, int64_t K, const void* x,
                       int64_t ldx, void* y, int32_t y_dtype, int64_t ldy, float* part, hipStream_t st) {
  if (y_dtype == kBF16) mxfp4_gemv_t<uint16_t>(B, packed, e8m0, N, K, x, ldx, y, ldy, part, st);
  else mxfp4_gemv_t<float>(B, packed, e8m0, N, K, x, ldx, y, ldy, part, st);
  const int S = mxfp4_gemv_splits(K, B);
  if (S > 1) launch_gemv_finalize(part, S, B, N, y, y_dtype, ldy, st);
}

}  // namespace gwb
