// Prefill GEMM on quantized weights: y[m, n] = sum_k x[m, k] * dequant(W)[n, k] for M
// rows of bf16 activations. Page export_gptq_cpu.py: vLLM's W4A16 kernels consume the
// GPTQ tensors as stored; page quantize_dflash_mxfp4.py serves its linears as MXFP4.
// The dequantized weights never reach memory: each wavefront turns its packed words
// into bf16 B operands of the matrix cores (v_mfma_f32_16x16x32_bf16, float32
// accumulation) in registers, and the activations are staged through LDS, shared by
// the block's four wavefronts.
//
// Block: 4 wavefronts, BM = 16*MT rows x 256 columns; wavefront w owns the 64 columns
// from nw = n0 + 64w and all BM rows (MT x 4 MFMA tiles of 16 x 16). Lane l (j = l % 16,
// q = l / 16) feeds B column j of tile t with the weights of column nw + 4j + t, so its
// accumulators hold rows 16mt + 4q + r (r < 4) of the 4 adjacent columns nw + 4j .. +3.
// K runs in stages of 128 through a double-buffered LDS tile of activations.
//
// GPTQ: codes c are integers and bf16(128 + c) is exact: a byte select and a mask turn
// codes 2i and 2i+1 of a word into such a pair. Per group the matrix cores sum
// T = sum_k x (128 + c) (exact products); the group adds s * (T - (128 + z) * sum_k x)
// to the output, with the group sums of x from a pre-pass (float64 sums, rounded once).
// A step covers 32 consecutive k, so a group ends on a step boundary for every group
// size.
// MXFP4: the scaled FP4 conversion gives the exact bf16 weights (E2M1 times
// 2^(e8m0 - 127)). A lane's 8-k slot in step s is k0 + 32q + 8s, so over a stage it
// covers one 32-block of each of its columns: one 16-byte load of codes and one scale
// byte per column and stage. A scale byte of 255 (no E8M0 value; the page's products
// are inf or NaN) is flagged in the loop and its columns recomputed after it.
//
// Activations go from memory straight to LDS (global_load_lds_dwordx4, no registers).
// The tile holds BM rows of 16 chunks (8 bf16 each) without padding; chunk kc of row r
// sits at slot 16r + (kc ^ swz(r & 15)). An operand read has 16 rows per 8-k chunk
// index and, across lane groups, chunk indices 4 apart (MXFP4) or 1 apart (GPTQ); the
// swizzle keeps the 32 lanes a read serves per pass on distinct banks in both cases
// (the plain r & 15 left MXFP4 reads 2-way conflicted). Rows past M and columns past N
// load clamped (valid) data whose results are not stored.
#include "kernels.hpp"
#include "mxfp4_math.hpp"
#include "uintx_layout.hpp"

namespace gwb {

typedef __bf16 gm_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float gm_f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGmBN = 256;            // columns per block
constexpr int kGmBK = 128;            // k per stage
constexpr int kGmSumMax = 4 * 128;    // group sums of one stage: up to 4 groups x BM rows

__device__ __forceinline__ gm_f32x4_t mfma_bf16(U4 a, U4 b, gm_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gm_bf16x8_t, a),
                                                  __builtin_bit_cast(gm_bf16x8_t, b), c, 0, 0, 0);
}

// Workgroups go round-robin over the 8 XCDs, each with its own L2. Each XCD gets a
// contiguous range of tiles; tiles run in bands of up to 4 row tiles across all column
// tiles, so the blocks an XCD holds at one time share activation rows and weights.
__device__ __forceinline__ void gemm_tile(int id, int gx, int gy, int& bx, int& by) {
  const int T = gx * gy, xcd = id & 7, rem = T & 7;
  const int t = xcd * (T >> 3) + min(xcd, rem) + (id >> 3);
  const int band = t / (4 * gy), first = band * 4, rows = min(4, gx - first);
  const int r = t - first * gy;
  bx = first + r % rows;
  by = r / rows;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// XOR applied to the chunk index of tile row r (r & 15 = j): a permutation of 0..15 in
// which rows of equal parity never differ by 1 or 4.
__device__ __forceinline__ int swz(int j) {
  const int i = j >> 1;
  return (((i & 4) << 1) | (i & 2) | ((i & 1) * 5)) ^ (j & 1);
}

// The activation tile's source offsets for this lane (elements from x + k0): wavefront
// w's i-th fill instruction writes slots (4i + w) * 64 .. +63, one per lane, i.e. row
// 16i + 4w + lane/16 at swizzled slot lane % 16.
template <int MT>
__device__ __forceinline__ void a_offsets(int64_t ldx, int M, int m0, int wv, int lane, uint32_t (&off)[MT]) {
  const int rr = 4 * wv + (lane >> 4), kc = (lane & 15) ^ swz(rr);
#pragma unroll
  for (int i = 0; i < MT; ++i) off[i] = (uint32_t)((int64_t)min(m0 + 16 * i + rr, M - 1) * ldx + 8 * kc);
}
template <int MT>
__device__ __forceinline__ void a_fetch(const uint32_t (&off)[MT], const uint16_t* xk, uint16_t* lds, int wv) {
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    // (a named pointer: the builtin given the sum directly fails to instantiate in
    // clang's host pass, which then silently drops the kernel's launch stub)
    const uint16_t* src = xk + off[i];
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(lds + (4 * i + wv) * 512), 16, 0, 0);
  }
}
// Element offset of the lane's operand chunk kc in row j of the first 16-row tile.
__device__ __forceinline__ int a_slot(int j, int kc) { return (16 * j + (kc ^ swz(j))) * 8; }

// Wait for this wavefront's outstanding memory loads (the LDS fills included), then
// for the whole block.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
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
// Codes 2i and 2i+1 of a word as bf16(128 + c) values of one dword: byte i of w and of
// w >> 4 into bytes 0 and 2, low nibbles kept, exponent bits of 128 added.
// e is held in a register by the caller: with both constants as operands the compiler
// cannot form one v_and_or_b32 (one scalar operand per instruction) and splits it.
__device__ __forceinline__ U4 gptq_pairs(uint32_t w, uint32_t e) {
  const uint32_t h = w >> 4, m = 0x000F000Fu;
  return U4{(__builtin_amdgcn_perm(h, w, 0x0C040C00u) & m) | e, (__builtin_amdgcn_perm(h, w, 0x0C050C01u) & m) | e,
            (__builtin_amdgcn_perm(h, w, 0x0C060C02u) & m) | e, (__builtin_amdgcn_perm(h, w, 0x0C070C03u) & m) | e};
}

template <bool SYM, int G, int MT, typename TY>
__global__ __launch_bounds__(256, MT <= 2 || (MT == 4 && G == 128) ? 2 : 1) void gptq_gemm_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int M, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ sc, const uint32_t* __restrict__ qz, int N, int K, const float* __restrict__ gsum,
    int Mp, TY* __restrict__ y, int64_t ldy, int gx, int gy, int S) {
  constexpr int BM = 16 * MT, SPG = G / 32, NGS = kGmBK / G;   // steps per group, groups per stage
  constexpr int SUMS = BM * NGS / 4;                            // 16-byte chunks of group sums per stage
  static_assert(SUMS <= 256 && BM * NGS <= kGmSumMax, "group sums of a stage fit one chunk per thread");
  // one LDS object: activation tiles, then group sums (with two objects the compiler
  // waits for every outstanding load before the stage's first LDS read)
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * BM * 128 + 2 * 2 * NGS * BM];
  uint16_t(*As)[BM * 128] = reinterpret_cast<uint16_t(*)[BM * 128]>(smem);
  float(*Ss)[NGS * BM] = reinterpret_cast<float(*)[NGS * BM]>(smem + 2 * BM * 128);

  // K split (small grids): block = split * tiles + tile; split s takes stages
  // [s * nst / S, (s + 1) * nst / S) and stores float32 partials at y + s * M * ldy
  const int T = gx * gy, split = (int)blockIdx.x / T, nst = K / kGmBK;
  const int st0 = split * nst / S, st1 = (split + 1) * nst / S;
  y += (int64_t)split * M * ldy;
  int bx, by;
  gemm_tile((int)blockIdx.x - split * T, gx, gy, bx, by);
  const int lane = threadIdx.x & 63, j = lane & 15, q = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int m0 = bx * BM, nl = by * kGmBN + wv * 64 + 4 * j;
  const bool nok = nl < N;
  const int nc = min(nl, N - 4);                     // clamped column for loads
  const int zsh = 4 * (nc & 7);
  const uint32_t qoff = (uint32_t)(q * N + nc);      // qweight words from row k0/8 + 4s
  const int p = wv * 64 + lane;                      // group-sum chunk of this thread (p < SUMS)
  const uint32_t soff = (uint32_t)((p / (BM / 4)) * Mp + m0 + 4 * (p % (BM / 4)));   // from row k0/G
  int aoff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) aoff[s] = a_slot(j, 4 * s + q);
  uint32_t aof[MT];
  a_offsets<MT>(ldx, M, m0, wv, lane, aof);
  uint32_t pe = 0x43004300u;
  asm volatile("" : "+v"(pe));   // keep the constant in a vector register

  U4 wv4[4];
  uint2 scv[NGS];
  uint32_t zv[NGS];
  // Each stage reads its group sums from LDS before it issues the next fills: an LDS
  // access behind a pending fill makes the compiler wait for all outstanding loads.
  auto fetch = [&](int k0, int buf) {
    a_fetch<MT>(aof, x + k0, As[buf], wv);
    if (p < SUMS) {
      const float* src = gsum + (int64_t)(k0 / G) * Mp + soff;
      __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(&Ss[buf][0] + wv * 256), 16, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) wv4[s] = ld16(qw + (int64_t)(k0 / 8 + 4 * s) * N + qoff);
#pragma unroll
    for (int gi = 0; gi < NGS; ++gi) {
      const int64_t g = k0 / G + gi;
      scv[gi] = *reinterpret_cast<const uint2*>(sc + g * N + nc);
      if constexpr (!SYM) zv[gi] = qz[g * (N / 8) + nc / 8];
    }
  };

  gm_f32x4_t acc[MT][4], tmp[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[mt][t] = gm_f32x4_t{0.f, 0.f, 0.f, 0.f};

  fetch(st0 * kGmBK, 0);
  stage_barrier();
  for (int st = st0; st < st1; ++st) {
    const int buf = (st - st0) & 1;
    const uint16_t* A = As[buf];
    float4 sx[NGS][MT];
#pragma unroll
    for (int gi = 0; gi < NGS; ++gi)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) sx[gi][mt] = *reinterpret_cast<const float4*>(&Ss[buf][gi * BM + 16 * mt + 4 * q]);
    U4 w[4];
    uint2 scl[NGS];
    uint32_t zl[NGS];
#pragma unroll
    for (int s = 0; s < 4; ++s) w[s] = wv4[s];
#pragma unroll
    for (int gi = 0; gi < NGS; ++gi) {
      scl[gi] = scv[gi];
      if constexpr (!SYM) zl[gi] = zv[gi];
    }
    if (st + 1 < st1) fetch((st + 1) * kGmBK, buf ^ 1);

#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const U4 b[4] = {gptq_pairs(w[s].x, pe), gptq_pairs(w[s].y, pe), gptq_pairs(w[s].z, pe),
                       gptq_pairs(w[s].w, pe)};
      if (s % SPG == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int t = 0; t < 4; ++t) tmp[mt][t] = gm_f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const U4 a = *reinterpret_cast<const U4*>(A + aoff[s] + 16 * mt * 128);
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
          else cz[t] = -(float)(128u + ((zl[gi] >> (zsh + 4 * t)) & 0xFu));
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const float sxa[4] = {sx[gi][mt].x, sx[gi][mt].y, sx[gi][mt].z, sx[gi][mt].w};
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[mt][t][r] = fmaf(sf[t], fmaf(cz[t], sxa[r], tmp[mt][t][r]), acc[mt][t][r]);
        }
      }
    }
    stage_barrier();
  }
  gemm_store<MT, TY>(acc, y, ldy, M, m0, q, nl, nok);
}

// ------------------------------------------------------------------ MXFP4
template <int MT, typename TY>
__global__ __launch_bounds__(256, 2) void mxfp4_gemm_kernel(const uint16_t* __restrict__ x, int64_t ldx, int M,
                                                           const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ e8m0, int N, int K,
                                                           TY* __restrict__ y, int64_t ldy, int gx, int gy,
                                                           int S) {
  constexpr int BM = 16 * MT;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * 128];

  // K split (small grids): block = split * tiles + tile; split s takes stages
  // [s * nst / S, (s + 1) * nst / S) and stores float32 partials at y + s * M * ldy
  const int T = gx * gy, split = (int)blockIdx.x / T, nst = K / kGmBK;
  const int st0 = split * nst / S, st1 = (split + 1) * nst / S;
  y += (int64_t)split * M * ldy;
  int bx, by;
  gemm_tile((int)blockIdx.x - split * T, gx, gy, bx, by);
  const int lane = threadIdx.x & 63, j = lane & 15, q = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int m0 = bx * BM, nl = by * kGmBN + wv * 64 + 4 * j;
  const bool nok = nl < N;
  const int nc = min(nl, N - 4);
  const int64_t rowb = K / 2, rowe = K / 32;
  const uint32_t coff = (uint32_t)(nc * rowb + 16 * q);   // codes of column nc from byte k0/2 (+ t rowb)
  const uint32_t eoff = (uint32_t)(nc * rowe + q);        // scale bytes from k0/32 (+ t rowe)
  int aoff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) aoff[s] = a_slot(j, 4 * q + s);
  uint32_t aof[MT];
  a_offsets<MT>(ldx, M, m0, wv, lane, aof);

  U4 wv4[4];
  uint32_t ev[4];
  auto fetch = [&](int k0, int buf) {
    a_fetch<MT>(aof, x + k0, As[buf], wv);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      wv4[t] = ld16(codes + (k0 / 2 + t * rowb) + coff);
      ev[t] = e8m0[(k0 / 32 + t * rowe) + eoff];
    }
  };

  gm_f32x4_t acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[mt][t] = gm_f32x4_t{0.f, 0.f, 0.f, 0.f};

  fetch(st0 * kGmBK, 0);
  stage_barrier();
  uint32_t nanc = 0;   // bit t: column nc + t has a block with scale byte 255
  for (int st = st0; st < st1; ++st) {
    const int buf = (st - st0) & 1;
    U4 w[4];
    uint32_t e[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      w[t] = wv4[t];
      e[t] = ev[t];
    }
    if (st + 1 < st1) fetch((st + 1) * kGmBK, buf ^ 1);
    float scl[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      scl[t] = mx_scale_operand(e[t]);
      nanc |= (uint32_t)(e[t] == 255u) << t;
    }
    const uint16_t* A = As[buf];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      U4 b[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t wd = s == 0 ? w[t].x : s == 1 ? w[t].y : s == 2 ? w[t].z : w[t].w;
        b[t] = U4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl[t], 0)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl[t], 1)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl[t], 2)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl[t], 3))};
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const U4 a = *reinterpret_cast<const U4*>(A + aoff[s] + 16 * mt * 128);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[mt][t] = mfma_bf16(a, b[t], acc[mt][t]);
      }
    }
    stage_barrier();
  }
  // Columns with a scale byte of 255 (no E8M0 value): the loop's products there are
  // meaningless, and the page's weights +-E2M1 * 2^128 are inf or NaN, so the output is
  // the float32 sum over those blocks alone (inf or NaN; adding the finite rest cannot
  // change it). Wave-uniform and rare; a plain loop over K.
  if (__any(nanc != 0u)) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (!((nanc >> t) & 1u)) continue;
      const uint8_t* crow = codes + (int64_t)(nc + t) * rowb;
      const uint8_t* erow = e8m0 + (int64_t)(nc + t) * rowe;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint16_t* xr = x + (int64_t)min(m0 + 16 * mt + 4 * q + r, M - 1) * ldx;
          float sum = 0.f;
          for (int blk = 0; blk < K / 32; ++blk) {
            if (erow[blk] != 255u) continue;
            for (int k = 32 * blk; k < 32 * blk + 32; ++k) {
              const uint32_t c = (crow[k >> 1] >> (4 * (k & 1))) & 0xFu;
              sum += bf16_to_f32(xr[k]) * mx_value_nan_scale(c);
            }
          }
          acc[mt][t][r] = sum;
        }
    }
  }
  gemm_store<MT, TY>(acc, y, ldy, M, m0, q, nl, nok);
}

// ------------------------------------------------------------------ launchers
// Block rows: two wavefronts per SIMD (at most 256 registers each) hide each other's
// waits and GPTQ's per-group VALU work; that holds for 128-row MXFP4 blocks and 64-row
// GPTQ blocks with 128-groups (measured at M = 2048: MXFP4 1150 vs 920 TFLOP/s for one
// wavefront per SIMD, GPTQ 930-970 vs 640). Smaller GPTQ groups keep 64 rows at one
// wavefront per SIMD (their per-group state does not fit 256 registers).

// K splits: small-M grids (one row tile over N / 256 column tiles) leave most CUs idle;
// up to 4 splits, each of at least 2 stages, bring the grid to about 512 blocks. Their
// float32 partials (M x N each) are summed in split order by a second kernel. Only for
// M <= 64, where the partials stay small next to the packed weight.
// 16-row granularity of the matrix-core tiles: small M takes 16- or 32-row blocks
// rather than computing padding rows.
static int gemm_small_mt(int64_t M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }
// K splits for M <= 64: enough workgroups for two per compute unit (512 with T tiles),
// each split at least 2 stages; up to 4 splits always, up to 16 while the partials
// (S M N float32, written and read back) stay within a quarter of the packed weight
// (N K / 2 bytes), i.e. S <= K / (32 M).
static int gemm_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t rows = 16 * gemm_small_mt(M);
  const int64_t T = ((M + rows - 1) / rows) * ((N + kGmBN - 1) / kGmBN), nst = K / kGmBK;
  if (M > 64 || T == 0) return 1;
  int64_t S = (512 + T - 1) / T;
  const int64_t cap = K / (32 * M) > 4 ? K / (32 * M) : 4;
  if (S > cap) S = cap;
  if (S > 16) S = 16;
  if (S > nst / 2) S = nst / 2;
  return S < 1 ? 1 : (int)S;
}
static size_t align256(size_t b) { return (b + 255) / 256 * 256; }
static size_t sums_bytes(bool gptq, int group, int64_t M, int64_t K) {
  if (!gptq) return 0;
  const int64_t Mp = (M + 127) / 128 * 128;
  return align256((size_t)(K / group) * (size_t)Mp * sizeof(float));
}

size_t gemm_workspace_bytes(bool gptq, int group, int64_t M, int64_t N, int64_t K) {
  const int S = gemm_splits(M, N, K);
  return sums_bytes(gptq, group, M, K) + (S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0);
}

// y[m, n] = sum over splits of part[s][m][n], in split order; 4 outputs per thread.
template <typename TY>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float* __restrict__ part, int S, int M, int N,
                                                         TY* __restrict__ y, int64_t ldy) {
  const int64_t MN = (int64_t)M * N, i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= MN) return;
  float4 v = *reinterpret_cast<const float4*>(part + i);
  for (int s = 1; s < S; ++s) {
    const float4 u = *reinterpret_cast<const float4*>(part + s * MN + i);
    v.x += u.x;
    v.y += u.y;
    v.z += u.z;
    v.w += u.w;
  }
  const int64_t m = i / N, n = i - m * N;
  TY* p = y + m * ldy + n;
  if constexpr (sizeof(TY) == 4) *reinterpret_cast<float4*>(p) = v;
  else *reinterpret_cast<uint2*>(p) = uint2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
}
static void gemm_reduce(const float* part, int S, int M, int N, void* y, int32_t y_dtype, int64_t ldy,
                        hipStream_t st) {
  const int64_t threads = (int64_t)M * N / 4;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (y_dtype == kF32)
    hipLaunchKernelGGL(gemm_reduce_kernel<float>, grid, dim3(256), 0, st, part, S, M, N, (float*)y, ldy);
  else
    hipLaunchKernelGGL(gemm_reduce_kernel<uint16_t>, grid, dim3(256), 0, st, part, S, M, N, (uint16_t*)y, ldy);
}

template <bool SYM, int G, int MT, typename TY>
static void gptq_gemm_go(const void* x, int64_t ldx, int M, const void* qw, const void* sc, const void* qz, int N,
                         int K, const float* gs, int Mp, void* y, int64_t ldy, int S, hipStream_t st) {
  const int gx = (M + 16 * MT - 1) / (16 * MT), gy = (N + kGmBN - 1) / kGmBN;
  hipLaunchKernelGGL((gptq_gemm_kernel<SYM, G, MT, TY>), dim3(gx * gy * S), dim3(256), 0, st, (const uint16_t*)x,
                     ldx, M, (const uint32_t*)qw, (const uint16_t*)sc, (const uint32_t*)qz, N, K, gs, Mp, (TY*)y, ldy,
                     gx, gy, S);
}
template <int G>
static void group_sums_go(const void* x, int64_t ldx, int M, int K, int Mp, float* sums, hipStream_t st) {
  const int64_t lanes = (int64_t)Mp * (K / 8);
  hipLaunchKernelGGL((gemm_group_sums_kernel<G>), dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, st,
                     (const uint16_t*)x, ldx, M, K, Mp, sums);
}
// GPTQ blocks are 64 rows (two wavefronts per SIMD with 128-groups); with K splits the
// kernel writes float32 partials and the reduction writes y.
template <bool SYM, int G, int MT>
static void gptq_gemm_mt(const void* x, int64_t ldx, int M, const void* qw, const void* sc, const void* qz, int N,
                         int K, float* sums, int Mp, void* y, int32_t y_dtype, int64_t ldy, float* part,
                         hipStream_t st) {
  const int S = gemm_splits(M, N, K);
  if (S > 1) {
    gptq_gemm_go<SYM, G, MT, float>(x, ldx, M, qw, sc, qz, N, K, sums, Mp, part, N, S, st);
    gemm_reduce(part, S, M, N, y, y_dtype, ldy, st);
  } else if (y_dtype == kBF16) {
    gptq_gemm_go<SYM, G, MT, uint16_t>(x, ldx, M, qw, sc, qz, N, K, sums, Mp, y, ldy, 1, st);
  } else {
    gptq_gemm_go<SYM, G, MT, float>(x, ldx, M, qw, sc, qz, N, K, sums, Mp, y, ldy, 1, st);
  }
}
template <bool SYM, int G>
static void gptq_gemm_run(const void* x, int64_t ldx, int M, const void* qw, const void* sc, const void* qz, int N,
                          int K, float* sums, int Mp, void* y, int32_t y_dtype, int64_t ldy, float* part,
                          hipStream_t st) {
  const int mt = gemm_small_mt(M);
  if (mt == 1) gptq_gemm_mt<SYM, G, 1>(x, ldx, M, qw, sc, qz, N, K, sums, Mp, y, y_dtype, ldy, part, st);
  else if (mt == 2) gptq_gemm_mt<SYM, G, 2>(x, ldx, M, qw, sc, qz, N, K, sums, Mp, y, y_dtype, ldy, part, st);
  else gptq_gemm_mt<SYM, G, 4>(x, ldx, M, qw, sc, qz, N, K, sums, Mp, y, y_dtype, ldy, part, st);
}

void launch_gptq_gemm(bool sym, int group, const void* qweight, const void* scales, const void* qzeros, int64_t N,
                      int64_t K, const void* x, int64_t M, int64_t ldx, void* y, int32_t y_dtype, int64_t ldy,
                      void* workspace, hipStream_t st) {
  const int Mp = (int)((M + 127) / 128 * 128);
  float* sums = (float*)workspace;
  float* part = (float*)((char*)workspace + sums_bytes(true, group, M, K));
#define GWB_GEMM_G(G)                                                                                               \
  do {                                                                                                              \
    group_sums_go<G>(x, ldx, (int)M, (int)K, Mp, sums, st);                                                         \
    if (sym) gptq_gemm_run<true, G>(x, ldx, (int)M, qweight, scales, qzeros, (int)N, (int)K, sums, Mp, y, y_dtype,  \
                                    ldy, part, st);                                                                 \
    else gptq_gemm_run<false, G>(x, ldx, (int)M, qweight, scales, qzeros, (int)N, (int)K, sums, Mp, y, y_dtype,     \
                                 ldy, part, st);                                                                    \
  } while (0)
  if (group == 32) GWB_GEMM_G(32);
  else if (group == 64) GWB_GEMM_G(64);
  else GWB_GEMM_G(128);
#undef GWB_GEMM_G
}

template <int MT, typename TY>
static void mxfp4_gemm_go(const void* x, int64_t ldx, int M, const void* codes, const void* e8, int N, int K,
                          void* y, int64_t ldy, int S, hipStream_t st) {
  const int gx = (M + 16 * MT - 1) / (16 * MT), gy = (N + kGmBN - 1) / kGmBN;
  hipLaunchKernelGGL((mxfp4_gemm_kernel<MT, TY>), dim3(gx * gy * S), dim3(256), 0, st, (const uint16_t*)x, ldx, M,
                     (const uint8_t*)codes, (const uint8_t*)e8, N, K, (TY*)y, ldy, gx, gy, S);
}

template <int MT>
static void mxfp4_gemm_mt(const void* packed, const void* e8m0, int64_t N, int64_t K, const void* x, int64_t M,
                          int64_t ldx, void* y, int32_t y_dtype, int64_t ldy, void* workspace, hipStream_t st) {
  const int S = gemm_splits(M, N, K);
  if (S > 1) {
    mxfp4_gemm_go<MT, float>(x, ldx, (int)M, packed, e8m0, (int)N, (int)K, workspace, N, S, st);
    gemm_reduce((const float*)workspace, S, (int)M, (int)N, y, y_dtype, ldy, st);
  } else if (y_dtype == kF32) {
    mxfp4_gemm_go<MT, float>(x, ldx, (int)M, packed, e8m0, (int)N, (int)K, y, ldy, 1, st);
  } else {
    mxfp4_gemm_go<MT, uint16_t>(x, ldx, (int)M, packed, e8m0, (int)N, (int)K, y, ldy, 1, st);
  }
}
// MXFP4 blocks are 128 rows above M = 64 (two wavefronts per SIMD either way).
void launch_mxfp4_gemm(const void* packed, const void* e8m0, int64_t N, int64_t K, const void* x, int64_t M,
                       int64_t ldx, void* y, int32_t y_dtype, int64_t ldy, void* workspace, hipStream_t st) {
  const int mt = M > 64 ? 8 : gemm_small_mt(M);
  if (mt == 1) mxfp4_gemm_mt<1>(packed, e8m0, N, K, x, M, ldx, y, y_dtype, ldy, workspace, st);
  else if (mt == 2) mxfp4_gemm_mt<2>(packed, e8m0, N, K, x, M, ldx, y, y_dtype, ldy, workspace, st);
  else if (mt == 4) mxfp4_gemm_mt<4>(packed, e8m0, N, K, x, M, ldx, y, y_dtype, ldy, workspace, st);
  else mxfp4_gemm_mt<8>(packed, e8m0, N, K, x, M, ldx, y, y_dtype, ldy, workspace, st);
}

// ------------------------------------------------------------------ uintx, bf16 weights
// Decode batches on the tiled uintx layout (page uintx_quant.py, forward). The flattened
// [N, K] weight is 8 segments of L1 = N K / 8 positions (segment t = rows t N/8 ..
// (t+1) N/8 - 1, position p = (row - t N/8) K + k); a shard byte holds position p of
// several segments (4-bit planes t & 3, nibble t >> 2; 2-bit planes t & 1, field t >> 1;
// 1-bit: bit t), so a lane takes the same positions of all 8 segments and every byte it
// loads serves all of them. Block: 16 activation rows x 64 positions-rows of each
// segment; wavefront w owns position-rows r = r0 + 16w .. +15, and lane l (j = l % 16,
// q = l / 16) feeds B column j of tile t (segment t) with row t N/8 + r0 + 16w + j over
// k0 + 32q .. +31: the MXFP4 kernel's k assignment, so the activation tile and its
// operand reads are shared with it. The B operands are the forward weights
// bf16((q - zp) s): c s - zp s is exact in float32 and one conversion rounds it, so every
// product with the bf16 activations is exact and the sums are float32. One 16-row tile
// converts each weight once per 16 activation rows: a decode kernel.
typedef __bf16 gm_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float gm_f32x2_t __attribute__((ext_vector_type(2)));
constexpr int kUxRows = 64;           // position-rows of each segment per block

__device__ __forceinline__ uint32_t ux_pair(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(gm_f32x2_t{a, b}, gm_bf16x2_t));
}
__device__ __forceinline__ uint32_t u4_word(const U4 (&v)[2], int i) {
  const U4& u = v[i >> 2];
  return (i & 3) == 0 ? u.x : (i & 3) == 1 ? u.y : (i & 3) == 2 ? u.z : u.w;
}

template <int NB, typename TY>
__global__ __launch_bounds__(256, 2) void uintx_gemm_kernel(const uint16_t* __restrict__ x, int64_t ldx, int M,
                                                           const uint8_t* __restrict__ packed,
                                                           const uint16_t* __restrict__ scales,
                                                           const uint8_t* __restrict__ zeros, Shards sh, int R8,
                                                           int K, int lg, TY* __restrict__ y, int64_t ldy, int gx,
                                                           int gy, int S) {
  using SB = ShardBits<NB>;
  constexpr int P4 = SB::has4 ? 4 : 0, P2 = SB::has2 ? 2 : 0, P1 = SB::has1 ? 1 : 0, NP = P4 + P2 + P1;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][16 * 128];

  const int T = gx * gy, split = (int)blockIdx.x / T, nst = K / kGmBK;
  const int st0 = split * nst / S, st1 = (split + 1) * nst / S;
  y += (int64_t)split * M * ldy;
  int bx, by;
  gemm_tile((int)blockIdx.x - split * T, gx, gy, bx, by);
  const int lane = threadIdx.x & 63, j = lane & 15, q = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int m0 = bx * 16, r = by * kUxRows + wv * 16 + j;
  const uint32_t L1 = (uint32_t)R8 * (uint32_t)K;
  const uint32_t pos = (uint32_t)min(r, R8 - 1) * (uint32_t)K + 32 * q;   // + k0: this lane's 32 positions
  uint32_t plane[NP];                    // byte offset of each shard plane in packed
#pragma unroll
  for (int i = 0; i < P4; ++i) plane[i] = (uint32_t)sh.base4 + i * L1;
#pragma unroll
  for (int i = 0; i < P2; ++i) plane[P4 + i] = (uint32_t)sh.base2 + i * L1;
  if constexpr (P1 != 0) plane[P4 + P2] = (uint32_t)sh.base1;
  int aoff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) aoff[s] = a_slot(j, 4 * q + s);
  uint32_t aof[1];
  a_offsets<1>(ldx, M, m0, wv, lane, aof);

  U4 pb[NP][2];
  uint32_t pq[8];                        // segment t's group: scale bits << 16 | zero point
  // uniform 64-bit bases plus 32-bit lane offsets (the scalar-base load form: no 64-bit
  // address arithmetic per load)
  const char* sbase = reinterpret_cast<const char*>(scales);
  auto fetch = [&](int k0, int buf) {
    a_fetch<1>(aof, x + k0, As[buf], wv);
    const uint8_t* pk = packed + k0;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const uint32_t o = plane[i] + pos;
      pb[i][0] = ld16(pk + o);
      pb[i][1] = ld16(pk + (o + 16u));
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t g = (t * L1 + pos + (uint32_t)k0) >> lg;
      pq[t] = ((uint32_t)*reinterpret_cast<const uint16_t*>(sbase + (g << 1)) << 16) | zeros[g];
    }
  };

  gm_f32x4_t acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = gm_f32x4_t{0.f, 0.f, 0.f, 0.f};

  fetch(st0 * kGmBK, 0);
  stage_barrier();
  for (int st = st0; st < st1; ++st) {
    const int buf = (st - st0) & 1;
    U4 b8[NP][2];
    uint32_t qp[8];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      b8[i][0] = pb[i][0];
      b8[i][1] = pb[i][1];
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) qp[t] = pq[t];
    if (st + 1 < st1) fetch((st + 1) * kGmBK, buf ^ 1);
    const uint16_t* A = As[buf];
    float sc[8], nzs[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      sc[t] = __uint_as_float(qp[t] & 0xFFFF0000u);
      nzs[t] = -((float)(qp[t] & 0xFFu) * sc[t]);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const U4 a = *reinterpret_cast<const U4*>(A + aoff[s]);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        uint32_t c[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int wi = 2 * s + h;                    // word of the lane's 32 bytes: k0 + 32q + 4 wi ..
          uint32_t v = 0u;
          if constexpr (SB::has4) v |= (u4_word(b8[t & 3], wi) >> (4 * (t >> 2))) & 0x0F0F0F0Fu;
          if constexpr (SB::has2) v |= ((u4_word(b8[P4 + (t & 1)], wi) >> (2 * (t >> 1))) & 0x03030303u) << SB::off2;
          if constexpr (SB::has1) v |= ((u4_word(b8[P4 + P2], wi) >> t) & 0x01010101u) << SB::off1;
          c[h] = v;
        }
        asm volatile("" : "+v"(c[0]), "+v"(c[1]));   // codes convert from their bytes (v_cvt_f32_ubyte0..3)
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = __builtin_fmaf((float)((c[e >> 2] >> (8 * (e & 3))) & 0xFFu), sc[t], nzs[t]);
        const U4 b = U4{ux_pair(f[0], f[1]), ux_pair(f[2], f[3]), ux_pair(f[4], f[5]), ux_pair(f[6], f[7])};
        acc[t] = mfma_bf16(a, b, acc[t]);
      }
    }
    stage_barrier();
  }
  if (r >= R8) return;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 4 * q + i;
      if (m >= M) continue;
      TY* p = y + (int64_t)m * ldy + (int64_t)t * R8 + r;
      if constexpr (sizeof(TY) == 4) *p = acc[t][i];
      else *p = (TY)(__float_as_uint(round_bf16(acc[t][i])) >> 16);
    }
}

// K splits toward 512 blocks (at most 32, each at least 2 stages, partials within a
// quarter of the packed weight as for the GEMM).
static int uintx_gemm_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t T = ((M + 15) / 16) * ((N / 8 + kUxRows - 1) / kUxRows), nst = K / kGmBK;
  if (T == 0) return 1;
  int64_t S = (512 + T - 1) / T;
  const int64_t cap = K / (32 * M) > 4 ? K / (32 * M) : 4;
  if (S > cap) S = cap;
  if (S > 32) S = 32;
  if (S > nst / 2) S = nst / 2;
  return S < 1 ? 1 : (int)S;
}
size_t uintx_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int S = uintx_gemm_splits(M, N, K);
  return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

template <int NB, typename TY>
static void uintx_gemm_go(const void* x, int64_t ldx, int M, const void* packed, const void* scales,
                          const void* zeros, int64_t N, int64_t K, int lg, void* y, int64_t ldy, int S,
                          hipStream_t st) {
  const int R8 = (int)(N / 8);
  const int gx = (M + 15) / 16, gy = (R8 + kUxRows - 1) / kUxRows;
  hipLaunchKernelGGL((uintx_gemm_kernel<NB, TY>), dim3(gx * gy * S), dim3(256), 0, st, (const uint16_t*)x, ldx, M,
                     (const uint8_t*)packed, (const uint16_t*)scales, (const uint8_t*)zeros, shards_of(NB, N * K),
                     R8, (int)K, lg, (TY*)y, ldy, gx, gy, S);
}
template <int NB>
static void uintx_gemm_nb(const void* x, int64_t ldx, int64_t M, const void* packed, const void* scales,
                          const void* zeros, int64_t N, int64_t K, int lg, void* y, int32_t y_dtype, int64_t ldy,
                          void* workspace, hipStream_t st) {
  const int S = uintx_gemm_splits(M, N, K);
  if (S > 1) {
    uintx_gemm_go<NB, float>(x, ldx, (int)M, packed, scales, zeros, N, K, lg, workspace, N, S, st);
    gemm_reduce((const float*)workspace, S, (int)M, (int)N, y, y_dtype, ldy, st);
  } else if (y_dtype == kF32) {
    uintx_gemm_go<NB, float>(x, ldx, (int)M, packed, scales, zeros, N, K, lg, y, ldy, 1, st);
  } else {
    uintx_gemm_go<NB, uint16_t>(x, ldx, (int)M, packed, scales, zeros, N, K, lg, y, ldy, 1, st);
  }
}
void launch_uintx_gemm(int nbits, int group, const void* packed, const void* scales, const void* zeros, int64_t N,
                       int64_t K, const void* x, int64_t M, int64_t ldx, void* y, int32_t y_dtype, int64_t ldy,
                       void* workspace, hipStream_t st) {
  const int lg = group == 32 ? 5 : (group == 64 ? 6 : 7);
  switch (nbits) {
    case 2: uintx_gemm_nb<2>(x, ldx, M, packed, scales, zeros, N, K, lg, y, y_dtype, ldy, workspace, st); break;
    case 3: uintx_gemm_nb<3>(x, ldx, M, packed, scales, zeros, N, K, lg, y, y_dtype, ldy, workspace, st); break;
    case 4: uintx_gemm_nb<4>(x, ldx, M, packed, scales, zeros, N, K, lg, y, y_dtype, ldy, workspace, st); break;
    case 5: uintx_gemm_nb<5>(x, ldx, M, packed, scales, zeros, N, K, lg, y, y_dtype, ldy, workspace, st); break;
    case 6: uintx_gemm_nb<6>(x, ldx, M, packed, scales, zeros, N, K, lg, y, y_dtype, ldy, workspace, st); break;
    default: uintx_gemm_nb<7>(x, ldx, M, packed, scales, zeros, N, K, lg, y, y_dtype, ldy, workspace, st); break;
  }
}

// ------------------------------------------------------------------ uintx decode
// Decode (B <= 8 activation rows) on the same layout, spread for memory parallelism
// rather than operand reuse: a wavefront takes 16 position-rows (lanes j) and one class
// of segments, those sharing their 4-bit plane (t & 3: segments t and t + 4) or, without
// a 4-bit shard, their 2-bit plane (t & 1: four segments), so it loads one plane of each
// shard present and keeps 2 or 4 accumulator tiles; the four wavefronts of a block cover
// all classes of 16 (or 32) position-rows. The block's activations for its K range sit
// in LDS for the whole kernel (one barrier, at the start), so wavefronts never wait for
// one another.
// A batch is 256 positions of each of the 16 rows: lane q holds the 16-byte pieces at
// 64u + 16q (u < 4) of each plane, so every load instruction reads 64 contiguous bytes
// of each row, and matrix-core step m takes positions 64 (m >> 1) + 16q + 8 (m & 1) to
// + 7 from lane q (any split of K into 32-k slices serves, with the activations read to
// match); the row's scales and zero points of the batch (256 / G groups, starting at a
// multiple of 256 / G) are one load each, so gwb_gemv takes this kernel only with the
// packed codes, scales and zero points 16-byte aligned. Measured on the 131072 x 2048
// head, 8 rows, 4 bits: 16 rows of 32 bytes per lane and batch, K bytes apart, 57 us; a
// contiguous 64-byte run per lane (each instruction reading 16 bytes every 64 of each
// row) 47 us; these pieces 42 us. Each wavefront keeps the next batch's codes, scales
// and zero points in flight while it converts and multiplies the current one.
template <int NB> struct UdShape {
  static constexpr int kSegs = (NB & 4) ? 2 : 4;   // segments per wavefront
  static constexpr int kClasses = 8 / kSegs;         // wavefronts per 16 position-rows
  static constexpr int kRowGroups = 4 / kClasses;    // 16-row groups per block
  static constexpr int kRun = 64;                    // bytes per lane, plane and batch
  static constexpr int kBatch = 4 * kRun;            // positions of a row per batch
};

template <int NB, int NGR>
struct UdBuf {
  static constexpr int W = UdShape<NB>::kRun / 16;   // 16-byte loads per plane
  U4 w4[W], w2[W], w1[W];                            // the lane's pieces of each plane
  uint32_t sb[UdShape<NB>::kSegs][(NGR + 1) / 2], zb[UdShape<NB>::kSegs][(NGR + 3) / 4];   // the row's scales, zero points
};

template <int NB, int G, typename TY>
__global__ __launch_bounds__(256) void uintx_decode_kernel(const uint16_t* __restrict__ x, int64_t ldx, int Bn,
                                                           const uint8_t* __restrict__ packed,
                                                           const uint16_t* __restrict__ scales,
                                                           const uint8_t* __restrict__ zeros, Shards sh, int R8, int K,
                                                           int kspan, TY* __restrict__ y, int64_t ldy,
                                                           float* __restrict__ part) {
  using SB = ShardBits<NB>;
  using SH = UdShape<NB>;
  constexpr int SEGS = SH::kSegs, RUN = SH::kRun, BP = SH::kBatch;
  constexpr int NGR = BP / G;                        // groups of a row in a batch
  constexpr int W = RUN / 16;
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // [Bn][kspan + 8]
  const int t = threadIdx.x, lane = t & 63, j = lane & 15, q = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int cls = wv % SH::kClasses, rg = wv / SH::kClasses;
  const int ks = (int)blockIdx.y * kspan, kend = min(K, ks + kspan);   // multiples of BP
  const int xp = kspan + 8;                      // LDS row pitch: 16 bytes of padding per row
  const uint16_t* xb = xs + min(j, Bn - 1) * xp + 16 * q - ks;   // rows past the batch repeat the last
  const int r = ((int)blockIdx.x * SH::kRowGroups + rg) * 16 + j;
  const uint32_t L1 = (uint32_t)R8 * (uint32_t)K;
  const uint32_t rowp = (uint32_t)min(r, R8 - 1) * (uint32_t)K;
  const uint32_t pos = rowp + 16 * q;   // rows past R8 read a valid row
  const uint32_t p4 = (uint32_t)sh.base4 + (uint32_t)(cls & 3) * L1 + pos;
  const uint32_t p2 = (uint32_t)sh.base2 + (uint32_t)(cls & 1) * L1 + pos;
  const uint32_t p1 = (uint32_t)sh.base1 + pos;
  auto seg = [&](int i) { return SB::has4 ? cls + 4 * i : cls + 2 * i; };
  const char* sbase = reinterpret_cast<const char*>(scales);
  auto load = [&](UdBuf<NB, NGR>& b, int k0) {
    const uint8_t* pk = packed + k0;
#pragma unroll
    for (int u = 0; u < W; ++u) {
      if constexpr (SB::has4) b.w4[u] = ld16(pk + (p4 + 64u * u));
      if constexpr (SB::has2) b.w2[u] = ld16(pk + (p2 + 64u * u));
      if constexpr (SB::has1) b.w1[u] = ld16(pk + (p1 + 64u * u));
    }
    // scale and zero point stay apart until the batch is converted: combining them here
    // would wait for both loads at once
#pragma unroll
    for (int i = 0; i < SEGS; ++i) {
      const uint32_t g = ((uint32_t)seg(i) * L1 + rowp + (uint32_t)k0) / (uint32_t)G;   // a multiple of NGR
      if constexpr (NGR == 8) {
        const U4 v = *reinterpret_cast<const U4*>(sbase + (g << 1));
        b.sb[i][0] = v.x; b.sb[i][1] = v.y; b.sb[i][2] = v.z; b.sb[i][3] = v.w;
        const uint2 z = *reinterpret_cast<const uint2*>(zeros + g);
        b.zb[i][0] = z.x; b.zb[i][1] = z.y;
      } else if constexpr (NGR == 4) {
        const uint2 v = *reinterpret_cast<const uint2*>(sbase + (g << 1));
        b.sb[i][0] = v.x; b.sb[i][1] = v.y;
        b.zb[i][0] = *reinterpret_cast<const uint32_t*>(zeros + g);
      } else {
        b.sb[i][0] = *reinterpret_cast<const uint32_t*>(sbase + (g << 1));
        b.zb[i][0] = *reinterpret_cast<const uint16_t*>(zeros + g);
      }
    }
  };
  gm_f32x4_t acc[SEGS];
#pragma unroll
  for (int i = 0; i < SEGS; ++i) acc[i] = gm_f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto word = [](const U4 (&v)[W], int wi) {
    const U4& u = v[wi >> 2];
    return (wi & 3) == 0 ? u.x : (wi & 3) == 1 ? u.y : (wi & 3) == 2 ? u.z : u.w;
  };
  const bool qhi = (q & 2) != 0;
  auto compute = [&](const UdBuf<NB, NGR>& b, int k0) {
#pragma unroll
    for (int m = 0; m < RUN / 8; ++m) {
      const U4 a = *reinterpret_cast<const U4*>(xb + k0 + 64 * (m >> 1) + 8 * (m & 1));
#pragma unroll
      for (int i = 0; i < SEGS; ++i) {
        const int tt = seg(i);
        // the group of positions 64 (m >> 1) + 16 q + 8 (m & 1) .. of the batch
        uint32_t swd, zwd;
        int hs, hz;
        if constexpr (G == 32) {
          const int g0 = 2 * (m >> 1);
          swd = b.sb[i][g0 >> 1];                      // groups g0, g0 + 1 in one word
          zwd = b.zb[i][g0 >> 2];
          hs = qhi ? 1 : 0;
          hz = (g0 & 3) + (qhi ? 1 : 0);
        } else {
          const int gi = G == 64 ? (m >> 1) : (m >> 2);
          swd = b.sb[i][gi >> 1];
          zwd = b.zb[i][gi >> 2];
          hs = gi & 1;
          hz = gi & 3;
        }
        const float scv = __uint_as_float(hs ? (swd & 0xFFFF0000u) : (swd << 16));
        const float nzv = -((float)((zwd >> (8 * hz)) & 0xFFu) * scv);
        uint32_t c[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int wi = 2 * m + h;
          uint32_t v = 0u;
          if constexpr (SB::has4) v |= (word(b.w4, wi) >> (4 * (tt >> 2))) & 0x0F0F0F0Fu;
          if constexpr (SB::has2) v |= ((word(b.w2, wi) >> (2 * (tt >> 1))) & 0x03030303u) << SB::off2;
          if constexpr (SB::has1) v |= ((word(b.w1, wi) >> tt) & 0x01010101u) << SB::off1;
          c[h] = v;
        }
        float f[8];
        if constexpr (NB <= 4) {
          // a code below 16 read as an OCP e4m3 byte is c * 2^-9 exactly: the scaled FP8
          // conversion at 2^9 gives two codes as floats per instruction
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const gm_f32x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c[h], 512.0f, false);
            const gm_f32x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c[h], 512.0f, true);
            f[4 * h] = lo[0]; f[4 * h + 1] = lo[1]; f[4 * h + 2] = hi[0]; f[4 * h + 3] = hi[1];
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = __builtin_fmaf(f[e], scv, nzv);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            f[e] = __builtin_fmaf((float)((c[e >> 2] >> (8 * (e & 3))) & 0xFFu), scv, nzv);
        }
        const U4 bw = U4{ux_pair(f[0], f[1]), ux_pair(f[2], f[3]), ux_pair(f[4], f[5]), ux_pair(f[6], f[7])};
        acc[i] = mfma_bf16(a, bw, acc[i]);
      }
      // one step at a time: left free, the scheduler converts many steps ahead of their
      // products and doubles the registers a wavefront needs
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Two batches per trip, one per buffer: load the next batch, then convert the current.
  // The loads are unconditional (past the last batch they re-read it), so the compiler
  // waits for exactly the current batch's loads and leaves the next batch's in flight;
  // after each group of loads, an empty asm with a memory clobber and a scheduling
  // barrier keep it from sinking the loads to their first use or hoisting the current
  // batch's arithmetic above them (either would wait for the loads at once).
  const int nbt = (kend - ks) / BP;
  UdBuf<NB, NGR> b0, b1;
  load(b0, ks);                                  // the weight stream starts before the staging
  asm volatile("" ::: "memory");
  stage_rows(xs, xp, x, ldx, Bn, ks, kend);
  __syncthreads();
  int bt = 0;
  for (; bt + 1 < nbt; bt += 2) {
    load(b1, ks + (bt + 1) * BP);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    compute(b0, ks + bt * BP);
    load(b0, ks + min(bt + 2, nbt - 1) * BP);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    compute(b1, ks + (bt + 1) * BP);
  }
  if (bt < nbt) compute(b0, ks + bt * BP);
  if (r >= R8) return;
  const int64_t N = 8 * (int64_t)R8;
#pragma unroll
  for (int i = 0; i < SEGS; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int b = 4 * q + e;
      if (b >= Bn) continue;
      const int64_t n = (int64_t)seg(i) * R8 + r;
      if (gridDim.y > 1) {
        part[((int64_t)blockIdx.y * Bn + b) * N + n] = acc[i][e];
      } else {
        TY* p = y + (int64_t)b * ldy + n;
        if constexpr (sizeof(TY) == 4) *p = acc[i][e];
        else *p = (TY)(__float_as_uint(round_bf16(acc[i][e])) >> 16);
      }
    }
}

// K splits: toward 1024 blocks (four wavefronts per SIMD), each split at least 2 batches,
// and the split's activations within kUdLds bytes of LDS.
constexpr int kUdLds = 64 * 1024;
template <int NB>
static int uintx_decode_blocks(int64_t N) {
  return (int)((N / 8 + 16 * UdShape<NB>::kRowGroups - 1) / (16 * UdShape<NB>::kRowGroups));
}
template <int NB>
static int uintx_decode_splits_nb(int64_t B, int64_t N, int64_t K) {
  constexpr int BP = UdShape<NB>::kBatch;
  const int blocks = uintx_decode_blocks<NB>(N);
  const int64_t nbt = K / BP;
  int64_t S = (1024 + blocks - 1) / blocks;
  if (S > nbt / 2) S = nbt / 2;
  if (S < 1) S = 1;
  while (S < nbt && (int64_t)B * ((nbt + S - 1) / S * BP + 8) * 2 > kUdLds) ++S;   // LDS bound
  const int64_t per = (nbt + S - 1) / S;                 // batches per split
  return (int)((nbt + per - 1) / per);                   // no split left empty
}
int uintx_decode_splits(int nbits, int64_t B, int64_t N, int64_t K) {
  switch (nbits) {
    case 2: return uintx_decode_splits_nb<2>(B, N, K);
    case 3: return uintx_decode_splits_nb<3>(B, N, K);
    case 4: return uintx_decode_splits_nb<4>(B, N, K);
    case 5: return uintx_decode_splits_nb<5>(B, N, K);
    case 6: return uintx_decode_splits_nb<6>(B, N, K);
    default: return uintx_decode_splits_nb<7>(B, N, K);
  }
}
size_t uintx_decode_workspace_bytes(int nbits, int64_t B, int64_t N, int64_t K) {
  const int S = uintx_decode_splits(nbits, B, N, K);
  return S > 1 ? (size_t)S * (size_t)B * (size_t)N * sizeof(float) : 0;
}

template <int NB, int G>
static void uintx_decode_nb(const void* x, int64_t ldx, int B, const void* packed, const void* scales,
                            const void* zeros, int64_t N, int64_t K, void* y, int32_t y_dtype, int64_t ldy,
                            void* workspace, hipStream_t st) {
  constexpr int BP = UdShape<NB>::kBatch;
  const int blocks = uintx_decode_blocks<NB>(N);
  const int S = uintx_decode_splits_nb<NB>(B, N, K);
  const int nbt = (int)(K / BP), kspan = (nbt + S - 1) / S * BP;
  const size_t lds = (size_t)B * (kspan + 8) * sizeof(uint16_t);
  const dim3 grid((unsigned)blocks, (unsigned)S);
  const Shards sh = shards_of(NB, N * K);
  if (S > 1) {
    hipLaunchKernelGGL((uintx_decode_kernel<NB, G, float>), grid, dim3(256), lds, st, (const uint16_t*)x, ldx, B,
                       (const uint8_t*)packed, (const uint16_t*)scales, (const uint8_t*)zeros, sh, (int)(N / 8),
                       (int)K, kspan, (float*)nullptr, (int64_t)0, (float*)workspace);
    launch_gemv_finalize((const float*)workspace, S, B, N, y, y_dtype, ldy, st);   // any y alignment
  } else if (y_dtype == kF32) {
    hipLaunchKernelGGL((uintx_decode_kernel<NB, G, float>), grid, dim3(256), lds, st, (const uint16_t*)x, ldx, B,
                       (const uint8_t*)packed, (const uint16_t*)scales, (const uint8_t*)zeros, sh, (int)(N / 8),
                       (int)K, kspan, (float*)y, ldy, (float*)nullptr);
  } else {
    hipLaunchKernelGGL((uintx_decode_kernel<NB, G, uint16_t>), grid, dim3(256), lds, st, (const uint16_t*)x, ldx,
                       B, (const uint8_t*)packed, (const uint16_t*)scales, (const uint8_t*)zeros, sh, (int)(N / 8),
                       (int)K, kspan, (uint16_t*)y, ldy, (float*)nullptr);
  }
}
template <int NB>
static void uintx_decode_g(int group, const void* x, int64_t ldx, int B, const void* packed, const void* scales,
                           const void* zeros, int64_t N, int64_t K, void* y, int32_t y_dtype, int64_t ldy,
                           void* workspace, hipStream_t st) {
  if (group == 32) uintx_decode_nb<NB, 32>(x, ldx, B, packed, scales, zeros, N, K, y, y_dtype, ldy, workspace, st);
  else if (group == 64) uintx_decode_nb<NB, 64>(x, ldx, B, packed, scales, zeros, N, K, y, y_dtype, ldy, workspace, st);
  else uintx_decode_nb<NB, 128>(x, ldx, B, packed, scales, zeros, N, K, y, y_dtype, ldy, workspace, st);
}
void launch_uintx_decode(int nbits, int group, const void* packed, const void* scales, const void* zeros, int64_t N,
                         int64_t K, const void* x, int64_t B, int64_t ldx, void* y, int32_t y_dtype, int64_t ldy,
                         void* workspace, hipStream_t st) {
  const int b = (int)B;
  switch (nbits) {
    case 2: uintx_decode_g<2>(group, x, ldx, b, packed, scales, zeros, N, K, y, y_dtype, ldy, workspace, st); break;
    case 3: uintx_decode_g<3>(group, x, ldx, b, packed, scales, zeros, N, K, y, y_dtype, ldy, workspace, st); break;
    case 4: uintx_decode_g<4>(group, x, ldx, b, packed, scales, zeros, N, K, y, y_dtype, ldy, workspace, st); break;
    case 5: uintx_decode_g<5>(group, x, ldx, b, packed, scales, zeros, N, K, y, y_dtype, ldy, workspace, st); break;
    case 6: uintx_decode_g<6>(group, x, ldx, b, packed, scales, zeros, N, K, y, y_dtype, ldy, workspace, st); break;
    default: uintx_decode_g<7>(group, x, ldx, b, packed, scales, zeros, N, K, y, y_dtype, ldy, workspace, st); break;
  }
}

}  // namespace gwb
