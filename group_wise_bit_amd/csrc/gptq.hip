// 4-bit GPTQ quantize+pack, unpack+dequantize and fused reconstruction error.
// Page export_gptq_cpu.py: pack_int32, quantize_sym (vLLM uint4b8, w = (code-8)*scale,
// qzeros all 7) and quantize_asym (zp stored as itself).
//
// A tile is 32 weight rows (output channels n) x 512 along K. Each lane takes 8
// consecutive k of one row (one 128-bit bf16 load), so a group of G is G/8 adjacent
// lanes while each load instruction of a wavefront reads 1 KB of one row (long DRAM
// runs). A group's extremes are reduced for all 8 rows of a wave at once, transposed
// over the group's lanes, so each (row, group) scale and zero point is computed by one
// lane (with IEEE division) and shared through LDS. A lane's 8 codes are one qweight
// word (r, n); words go through LDS so that the [K/8, N] int32 output leaves as 128-byte
// runs along n.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gwb {

// ------------------------------------------------------------- group extremes
// Order-preserving float keys of a lane's 8 weights. A 32-bit word holding two bf16
// weights, read as a float32, orders like its upper weight: the lower weight only adds
// mantissa bits below the upper one's last place, so words whose upper weights differ
// never swap. The word rotated by 16 bits orders like its lower weight. Clearing the
// low 16 bits of the extreme key gives that weight exactly. float32 weights are their
// own keys.
template <typename TIn> struct GqKeys;
template <> struct GqKeys<uint16_t> {
  static __device__ __forceinline__ void get(const Raw8<uint16_t>& r, float* o) {
    const uint32_t w[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] = __uint_as_float(w[i]);
      o[i + 4] = __uint_as_float((w[i] >> 16) | (w[i] << 16));
    }
  }
  static __device__ __forceinline__ float value(float k) { return __uint_as_float(__float_as_uint(k) & 0xFFFF0000u); }
};
template <> struct GqKeys<float> {
  static __device__ __forceinline__ void get(const Raw8<float>& r, float* o) { to_f32(r, o); }
  static __device__ __forceinline__ float value(float k) { return k; }
};

// One butterfly step over the first NV values: lanes with `up` set keep the upper half
// and send the lower, their partner (which has `up` clear) does the opposite.
template <int CTRL, int NV, bool MAX>
__device__ __forceinline__ void xstep(float (&v)[8], bool up) {
#pragma unroll
  for (int i = 0; i < NV / 2; ++i) {
    const float keep = up ? v[i + NV / 2] : v[i], send = up ? v[i] : v[i + NV / 2];
    const float other = dpp_read<CTRL>(send);
    v[i] = MAX ? fmaxf(keep, other) : fminf(keep, other);
  }
}

// Reduce 8 rows' values over the L lanes of a group, transposed: with LL = min(L, 8)
// and R = 8 / LL, lane l ends holding rows (l % LL) * R + j, j < R, in v[j]. The
// half-mirror partner of lane i is 7 - i, which differs in bit 2 (and in bits 0-1, which
// no earlier step has used); the quad steps pair lanes differing in bit 1, then bit 0;
// for 16 lanes a rotation by 8 joins the two half-rows, which hold the same rows.
template <int L, bool MAX>
__device__ __forceinline__ void xreduce(float (&v)[8], int lane) {
  static_assert(L == 4 || L == 8 || L == 16, "groups of 32, 64 or 128");
  if constexpr (L >= 8) {
    xstep<kDppHalfMirror, 8, MAX>(v, lane & 4);
    xstep<kDppXor2, 4, MAX>(v, lane & 2);
    xstep<kDppXor1, 2, MAX>(v, lane & 1);
    if constexpr (L == 16) {
      const float other = dpp_read<kDppRor8>(v[0]);
      v[0] = MAX ? fmaxf(v[0], other) : fminf(v[0], other);
    }
  } else {
    xstep<kDppXor2, 8, MAX>(v, lane & 2);
    xstep<kDppXor1, 4, MAX>(v, lane & 1);
  }
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

// Codes: with y the hardware reciprocal of s (within 1 ulp of 1/s) and t = x / s,
// u = fma(x, y, zp) is within (|t| + 8) * 1.5 * 2^-23 of t + zp, and fl(x / s) within
// |t| * 2^-24 of t. When every |u - rint(u)| of a lane's 8 weights stays below
// 0.5 - (A / s + 16) * 2^-19 (A the group's largest magnitude, so |t| <= A / s), t + zp
// and fl(x / s) + zp lie strictly inside the same unit interval around rint(u), so
// rint(u) = rint(fl(x / s)) + zp. Otherwise (the exact and near ties, a few weights in
// a thousand for bf16 data, or every weight of a group whose A / s reaches 2^18) the
// weight is divided exactly.
// SNR: also the reconstruction sums of the stored values, (c - z) times the fp16 scale
// as the dequantize kernel forms them, over the tile's valid weights; one partial pair
// per block (block = tile).
template <bool SYM, int G, typename TIn, bool SNR>
__global__ __launch_bounds__(256) void gptq_quant_kernel(const TIn* __restrict__ W, int64_t ldw,
                                                         int N, int K, int ntk,
                                                         uint32_t* __restrict__ qweight,
                                                         _Float16* __restrict__ scales,
                                                         uint32_t* __restrict__ qzeros,
                                                         int32_t* __restrict__ g_idx, double* __restrict__ part) {
  using T = TileG<G>;
  constexpr int L = T::L, LL = L < 8 ? L : 8, R = 8 / LL;
  __shared__ uint32_t qtile[kTR * kQS];
  __shared__ float4 qp[kTN][T::NG];                 // per tile row and group: {1/s, zp, margin, s}
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  // consecutive blocks take consecutive column tiles of one k range, so the qweight rows
  // they write (128 bytes each) lie side by side in memory
  const int ntn = (N + kTN - 1) / kTN;
  const int kt = blockIdx.x / ntn, nt = blockIdx.x - kt * ntn;
  (void)ntk;
  const int n0 = nt * kTN, k0 = kt * kTK;
  // Lanes past K read a valid place instead: K % G == 0, so their groups lie wholly past
  // K and every reduction below stays within one group. Rows past N repeat row N - 1.
  // Nothing of either reaches memory.
  const int kc = min(k0 + lane * 8, K - 8);
  Raw8<TIn> raw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) raw[i] = load_raw8(W + (int64_t)min(n0 + wave * 8 + i, N - 1) * ldw + kc);

  float lo[8], hi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float key[8];
    GqKeys<TIn>::get(raw[i], key);
    if constexpr (SYM) {
      float m = fabsf(key[0]);
#pragma unroll
      for (int j = 1; j < 8; ++j) m = fmaxf(m, fabsf(key[j]));
      hi[i] = m;
    } else {
      float a = key[0], b = key[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) {
        a = fminf(a, key[j]);
        b = fmaxf(b, key[j]);
      }
      lo[i] = a;
      hi[i] = b;
    }
  }
  if constexpr (!SYM) xreduce<L, false>(lo, lane);
  xreduce<L, true>(hi, lane);
  int big = 0;
  if (L < 16 || (lane & 8) == 0) {                  // for 16 lanes, lanes 8-15 repeat 0-7
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int row = (lane % LL) * R + j;
      float s, zp, a;
      if constexpr (SYM) {
        a = GqKeys<TIn>::value(hi[j]);
        s = fmaxf(a * 0.125f, 1e-9f);               // amax / 8: exact scaling by 2^-3
        zp = 8.0f;
      } else {
        const float mn = GqKeys<TIn>::value(lo[j]), mx = GqKeys<TIn>::value(hi[j]);
        s = fmaxf(mx - mn, 1e-9f) / 15.0f;
        zp = __builtin_amdgcn_fmed3f(rintf(-mn / s), 0.0f, 15.0f);
        a = fmaxf(fabsf(mn), fabsf(mx));
      }
      float y = __builtin_amdgcn_rcpf(s);
      float margin = 0.5f - __builtin_fmaf(a, y, 16.0f) * 0x1p-19f;
      if (!(margin > 0.0f)) {   // quotients up to 2^18 or beyond: every weight divides
        y = 0.0f;               // (u = zp then, so no overflow reaches the margin test)
        margin = -1.0f;
      }
      qp[wave * 8 + row][lane / L] = make_float4(y, zp, margin, s);
      if constexpr (SNR) {
        const float s16 = (float)(_Float16)s;
        big |= !(a < (sizeof(TIn) == 2 ? kSafeSqMax64 : kSafeSqMax)) || !__builtin_isfinite(s16) || s16 == 0.0f;
      }
    }
  }
  // one flag per tile: a group too large for the float32 squares of the fused
  // reconstruction sums, or whose fp16 scale overflowed or underflowed, sends the whole
  // tile through the float64 squares and the plain (c - z) * s
  bool tile_big = false;
  if constexpr (SNR) {
    tile_big = __syncthreads_or(big) != 0;
  } else {
    (void)big;
    __syncthreads();
  }
  const int gl = lane / L;
  double sw = 0.0, se = 0.0;
  float fa = 0.0f, fb = 0.0f;                  // bf16 weights: the lane's float32 sums over its 8 rows
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 p = qp[wave * 8 + i][gl];
    float x[8], u[8], c[8], dev = 0.0f;
    to_f32(raw[i], x);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u[j] = __builtin_fmaf(x[j], p.x, p.y);
      c[j] = rintf(u[j]);
      dev = fmaxf(dev, fabsf(u[j] - c[j]));
    }
    // Bf16 weights make exact and near ties x / s = k + 1/2 common (a few per thousand):
    // only the weights that fail the margin divide, each under its own mask. Symmetric
    // groups of bf16 weights with s = amax / 8 (exact) need no division: x / s = 8x / amax
    // is a ratio of 8-bit significands, which lies either exactly on a half step or at
    // least 1/510 away from every half step, far outside the margin band; so a weight
    // that fails the margin is an exact tie, x / s + 8 = u's nearest half step h, and the
    // page's rint(x / s) + 8 is rint(h) (8 is even).
    if (dev >= p.z) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (fabsf(u[j] - c[j]) >= p.z) {
          if (SYM && sizeof(TIn) == 2 && p.w != 1e-9f) c[j] = rintf(c[j] + copysignf(0.5f, u[j] - c[j]));
          else c[j] = rintf(x[j] / p.w) + p.y;
        }
    }
    uint32_t ev = 0, od = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ev = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_amdgcn_fmed3f(c[2 * j], 0.0f, 15.0f), j, ev);
      od = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_amdgcn_fmed3f(c[2 * j + 1], 0.0f, 15.0f), j, od);
    }
    qtile[lane * kQS + wave * 8 + i] = ev | (od << 4);
    if constexpr (SNR) {
      if (n0 + wave * 8 + i < N && k0 + lane * 8 < K) {
        const float s16 = (float)(_Float16)p.w;
        float d[8];
        if (!tile_big) {
          // (c - z) * s is exact in float32 for a finite non-zero fp16 scale, so
          // c*s - z*s as one fma rounds it exactly
          const float nzs = -(p.y * s16);
#pragma unroll
          for (int j = 0; j < 8; ++j) d[j] = __builtin_fmaf(__builtin_amdgcn_fmed3f(c[j], 0.0f, 15.0f), s16, nzs);
          if constexpr (sizeof(TIn) == 2) acc_err8_f32_bf16_into(raw[i].v, x, d, fa, fb);
          else acc_err8_f32(x, d, sw, se);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) d[j] = (__builtin_amdgcn_fmed3f(c[j], 0.0f, 15.0f) - p.y) * s16;
          acc_err8(x, d, sw, se);
        }
      }
    }
  }
  if constexpr (SNR) block_sum2_store<256>(sw + (double)fa, se + (double)fb, part);   // synchronizes the block too
  __syncthreads();
  // qweight [K/8, N]: 64 r-rows x 32 words. Each store instruction of a wavefront writes
  // eight whole 128-byte rows (16 bytes per lane): non-temporal stores reach memory as
  // full lines (the packed tensors are read back much later, if at all, and ordinary
  // stores would leave them as dirty lines for the next kernel to write back).
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = wave * 16 + h * 8 + (lane >> 3), c4 = (lane & 7) * 4;
    if (k0 / 8 + r < K / 8 && n0 + c4 < N) {    // N % 8 == 0: a run that starts inside N ends inside it
      const uint32_t* src = &qtile[r * kQS + c4];
      st16_nt(qweight + (int64_t)(k0 / 8 + r) * N + n0 + c4, U4{src[0], src[1], src[2], src[3]});
    }
  }
  for (int e = t; e < T::NG * kTN; e += 256) {   // scales [K/G, N]
    const int g = e / kTN, rl = e % kTN;
    if (k0 + g * G < K && n0 + rl < N) scales[(int64_t)(k0 / G + g) * N + n0 + rl] = (_Float16)qp[rl][g].w;
  }
  static_assert(T::NG * (kTN / 8) <= 256, "one qzeros word per thread");
  if (t < T::NG * (kTN / 8)) {   // qzeros [K/G, N/8]
    const int g = t / (kTN / 8), q = t % (kTN / 8);
    if (k0 + g * G < K && n0 + 8 * q < N) {
      uint32_t w = 0x77777777u;
      if constexpr (!SYM) {
        w = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) w |= (uint32_t)qp[8 * q + i][g].y << (4 * i);
      }
      qzeros[(int64_t)(k0 / G + g) * (N / 8) + n0 / 8 + q] = w;
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
  __shared__ uint16_t stile[T::NG * kTN];          // fp16 scale bits, widened on use
  __shared__ uint32_t ztile[T::NG * (kTN / 8)];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const uint16_t* scale_bits = reinterpret_cast<const uint16_t*>(scales);
  double sw = 0.0, se = 0.0;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int nt = tile / ntk, kt = tile - nt * ntk;
    const int n0 = nt * kTN, k0 = kt * kTK;
    // Staging loads first, then the error sink's weights: the LDS stores below wait only
    // for the staging data, and the weights stay in flight across the barrier. (Rows
    // past N or k past K read clamped in-bounds places; those values are not used.)
    // each load instruction of a wavefront reads eight whole 128-byte qweight rows
    U4 qv[2];
    bool qok[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = wave * 16 + h * 8 + (lane >> 3), c4 = (lane & 7) * 4;
      qok[h] = k0 / 8 + r < K / 8 && n0 + c4 < N;    // N % 8 == 0: whole 16-byte runs
      qv[h] = qok[h] ? ld16_nt(qweight + (int64_t)(k0 / 8 + r) * N + n0 + c4) : U4{};
    }
    constexpr int kSPer = (T::NG * kTN + 255) / 256;   // scales per thread
    uint16_t sv[kSPer];
#pragma unroll
    for (int q = 0; q < kSPer; ++q) {
      const int e = t + 256 * q, gl = e / kTN, rl = e % kTN;
      sv[q] = 0;
      if (e < T::NG * kTN && k0 + gl * G < K && n0 + rl < N) sv[q] = scale_bits[(int64_t)(k0 / G + gl) * N + n0 + rl];
    }
    uint32_t zv = 0;
    if (!SYM && t < T::NG * (kTN / 8)) {
      const int gl = t / (kTN / 8), q = t % (kTN / 8);
      if (k0 + gl * G < K && n0 + 8 * q < N) zv = qzeros[(int64_t)(k0 / G + gl) * (N / 8) + n0 / 8 + q];
    }
    Raw8<TW> wr[8];
    if constexpr (SINK == kErr) {
      const int kc = min(k0 + lane * 8, K - 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) wr[i] = load_raw8(W + (int64_t)min(n0 + wave * 8 + i, N - 1) * ldw + kc);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (qok[h]) {
        uint32_t* dst = &qtile[(wave * 16 + h * 8 + (lane >> 3)) * kQS + (lane & 7) * 4];
        dst[0] = qv[h].x; dst[1] = qv[h].y; dst[2] = qv[h].z; dst[3] = qv[h].w;
      }
    }
#pragma unroll
    for (int q = 0; q < kSPer; ++q)
      if (t + 256 * q < T::NG * kTN) stile[t + 256 * q] = sv[q];
    if (!SYM && t < T::NG * (kTN / 8)) ztile[t] = zv;
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
          const float s = (float)__builtin_bit_cast(_Float16, stile[gl * kTN + rl]);
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
static int ntk_of(int64_t K) { return (int)((K + kTK - 1) / kTK); }
static unsigned tiles_of(int64_t N, int64_t K) { return (unsigned)(((N + kTN - 1) / kTN) * ntk_of(K)); }

template <bool SYM, int G, bool SNR>
static void quant_g(const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw, void* qw,
                    void* sc, void* qz, void* gi, double* part, hipStream_t st) {
  const dim3 grid(tiles_of(N, K));
  if (w_dtype == kBF16)
    hipLaunchKernelGGL((gptq_quant_kernel<SYM, G, uint16_t, SNR>), grid, dim3(256), 0, st, (const uint16_t*)W,
                       ldw, (int)N, (int)K, ntk_of(K), (uint32_t*)qw, (_Float16*)sc, (uint32_t*)qz, (int32_t*)gi,
                       part);
  else
    hipLaunchKernelGGL((gptq_quant_kernel<SYM, G, float, SNR>), grid, dim3(256), 0, st, (const float*)W, ldw,
                       (int)N, (int)K, ntk_of(K), (uint32_t*)qw, (_Float16*)sc, (uint32_t*)qz, (int32_t*)gi,
                       part);
}

template <bool SYM, bool SNR>
static void quant_s(int group, const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw,
                    void* qw, void* sc, void* qz, void* gi, double* part, hipStream_t st) {
  if (group == 32) quant_g<SYM, 32, SNR>(W, w_dtype, N, K, ldw, qw, sc, qz, gi, part, st);
  else if (group == 64) quant_g<SYM, 64, SNR>(W, w_dtype, N, K, ldw, qw, sc, qz, gi, part, st);
  else quant_g<SYM, 128, SNR>(W, w_dtype, N, K, ldw, qw, sc, qz, gi, part, st);
}

void launch_gptq_quant(bool sym, int group, const void* W, int32_t w_dtype, int64_t N, int64_t K,
                       int64_t ldw, void* qweight, void* scales, void* qzeros, void* g_idx,
                       hipStream_t st) {
  if (sym) quant_s<true, false>(group, W, w_dtype, N, K, ldw, qweight, scales, qzeros, g_idx, nullptr, st);
  else quant_s<false, false>(group, W, w_dtype, N, K, ldw, qweight, scales, qzeros, g_idx, nullptr, st);
}

// One partial pair per tile: only while the tiles fit the error kernel's partials.
bool gptq_quant_snr_fits(int group, int64_t N, int64_t K) { return tiles_of(N, K) == gptq_err_blocks(group, N, K); }
void launch_gptq_quant_snr(bool sym, int group, const void* W, int32_t w_dtype, int64_t N, int64_t K,
                           int64_t ldw, void* qweight, void* scales, void* qzeros, void* g_idx, double* part,
                           hipStream_t st) {
  if (sym) quant_s<true, true>(group, W, w_dtype, N, K, ldw, qweight, scales, qzeros, g_idx, part, st);
  else quant_s<false, true>(group, W, w_dtype, N, K, ldw, qweight, scales, qzeros, g_idx, part, st);
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
