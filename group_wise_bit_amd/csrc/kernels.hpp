// Internal launchers of libgwb (host side). Arguments have been validated by the
// C ABI layer (api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gwb {

constexpr int kF32 = 0;   // gwb_dtype values
constexpr int kBF16 = 1;
constexpr int kF16 = 2;
constexpr int kStore = 0;  // dequant sinks
constexpr int kErr = 1;

// Grid caps: streaming kernels loop over their units grid-stride. The error kernels
// keep their block count (and so their partial-sum layout and workspace) fixed by the
// shape alone, independent of the device.
constexpr unsigned kStreamGridCap = 1u << 20;
constexpr unsigned kErrGridCap = 1024;

// Blocks of 256 threads for a grid-stride streaming kernel over `units` thread-units:
// one unit per thread at most, and at most GWB_BLOCKS_PER_CU (default 8) blocks per
// compute unit of the current device. Launch time only (queries the device).
unsigned stream_blocks(uint64_t units);
// The same with per_cu blocks per compute unit (0: the default 8).
unsigned stream_grid(uint64_t units, int per_cu);
inline unsigned err_blocks_for(uint64_t units) {
  uint64_t g = (units + 255) / 256;
  return (unsigned)(g < kErrGridCap ? (g ? g : 1) : kErrGridCap);
}

// ---- MXFP4 (mxfp4.hip)
// part != NULL: also the reconstruction sums' per-block partials (mxfp4_err_blocks of them)
void launch_mxfp4_quant(bool page_ties, const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw,
                        void* packed, void* e8m0, double* part, hipStream_t st);
void launch_mxfp4_dequant(const void* packed, const void* e8m0, int64_t N, int64_t K, void* out,
                          int32_t out_dtype, int64_t ldo, hipStream_t st);
unsigned mxfp4_err_blocks(int64_t N, int64_t K);
void launch_mxfp4_err(const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw,
                      const void* packed, const void* e8m0, double* part, hipStream_t st);

// ---- GPTQ (gptq.hip); sym selects uint4b8, otherwise asymmetric with stored zp
void launch_gptq_quant(bool sym, int group, const void* W, int32_t w_dtype, int64_t N, int64_t K,
                       int64_t ldw, void* qweight, void* scales, void* qzeros, void* g_idx,
                       hipStream_t st);
void launch_gptq_dequant(bool sym, int group, const void* qweight, const void* scales,
                         const void* qzeros, int64_t N, int64_t K, void* out, int32_t out_dtype,
                         int64_t ldo, hipStream_t st);
unsigned gptq_err_blocks(int group, int64_t N, int64_t K);
// quantize and the reconstruction sums in one pass (gptq_err_blocks partials), when
// gptq_quant_snr_fits: one partial per tile
bool gptq_quant_snr_fits(int group, int64_t N, int64_t K);
void launch_gptq_quant_snr(bool sym, int group, const void* W, int32_t w_dtype, int64_t N, int64_t K,
                           int64_t ldw, void* qweight, void* scales, void* qzeros, void* g_idx, double* part,
                           hipStream_t st);
void launch_gptq_err(bool sym, int group, const void* W, int32_t w_dtype, int64_t N, int64_t K,
                     int64_t ldw, const void* qweight, const void* scales, const void* qzeros,
                     double* part, hipStream_t st);

// ---- GPTQ with act-order groups (gptq_act.hip): group of channel k = g_idx[k]; the tile
// kernels hold every group of a 32-row band in LDS (K/G <= kActMaxGroups) and quantization
// holds one weight row in LDS (K * element size <= kActMaxRowBytes)
constexpr int kActMaxGroups = 256;
constexpr int64_t kActMaxRowBytes = 65536;
size_t gptq_act_workspace_bytes(int64_t N, int64_t K, int group);
void launch_gptq_act_quant(bool sym, int group, const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw,
                           const int32_t* perm, void* qweight, void* scales, void* qzeros, int32_t* g_idx,
                           void* workspace, hipStream_t st);
void launch_gptq_act_dequant(bool sym, int group, const void* qweight, const void* scales, const void* qzeros,
                             const int32_t* g_idx, int64_t N, int64_t K, void* out, int32_t out_dtype, int64_t ldo,
                             hipStream_t st);
unsigned gptq_act_err_blocks(int64_t N, int64_t K);
void launch_gptq_act_err(bool sym, int group, const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw,
                         const void* qweight, const void* scales, const void* qzeros, const int32_t* g_idx,
                         double* part, hipStream_t st);
// act-order tensors into group order (perm: the channel at each position; status 0 ok,
// 1 a group without exactly G channels, 2 g_idx out of range), and the activation gather
// that the GEMV on group-ordered tensors starts with
void launch_gptq_group_order(int group, const void* qweight, const int32_t* g_idx, int64_t N, int64_t K,
                             void* qweight_out, int32_t* perm, int32_t* status, hipStream_t st);
void launch_gather_columns(const void* x, int64_t ldx, int64_t B, int64_t K, const int32_t* perm, void* xo,
                           hipStream_t st);

// ---- UINTX: tiled kernels (uintx_tiled.hpp) when N*K % (8 group) == 0, instantiated
// for bf16 group 64 in uintx.hip and for the other (dtype, group) pairs in uintx_bf16.hip,
// uintx_f16.hip, uintx_f32.hip; uintx_flat.hip for every other shape. dt is the weight
// dtype (kBF16, kF16, kF32); group 32, 64 or 128.
bool uintx_tiled(int32_t dt, int group, int64_t N, int64_t K);
size_t uintx_code_workspace(int32_t dt, int group, int64_t N, int64_t K);
// part != NULL (tiled layout only: uintx_tiled): also the reconstruction sums' per-block
// partials, uintx_err_blocks of them
void launch_uintx_quant(int nbits, int32_t dt, int group, const void* W, int64_t N, int64_t K, int64_t ldw,
                        void* packed, void* scales, void* zeros, void* workspace, double* part, hipStream_t st);
void launch_uintx_dequant(int nbits, int32_t dt, int group, const void* packed, const void* scales,
                          const void* zeros, int64_t N, int64_t K, void* out, int32_t out_dtype, int64_t ldo,
                          hipStream_t st);
unsigned uintx_err_blocks(int32_t dt, int group, int64_t N, int64_t K);
void launch_uintx_err(int nbits, int32_t dt, int group, const void* W, int64_t N, int64_t K, int64_t ldw,
                      const void* packed, const void* scales, const void* zeros, double* part, hipStream_t st);
void launch_uintx_quant_flat(int nbits, int32_t dt, int group, const void* W, int64_t N, int64_t K, int64_t ldw,
                             void* packed, void* scales, void* zeros, void* workspace, hipStream_t st);
void launch_uintx_dequant_flat(int nbits, int32_t dt, int group, const void* packed, const void* scales,
                               const void* zeros, int64_t N, int64_t K, void* out, int32_t out_dtype, int64_t ldo,
                               hipStream_t st);
unsigned uintx_flat_err_blocks(int64_t N, int64_t K);
// Where a GEMV's row sums go: K-split partials, or y itself (float32 or bf16, RNE).
struct GemvOut {
  enum { kPart = 0, kF32 = 1, kBF16 = 2 };
  float* part;
  void* y;
  int64_t ldy;
  int mode;
};
#define GWB_UINTX_TILED_DT(SUF)                                                                                     \
  void uintx_tiled_quant_##SUF(int nbits, int group, const void* W, int64_t N, int64_t K, int64_t ldw,              \
                               void* packed, void* scales, void* zeros, double* part, hipStream_t st);               \
  void uintx_tiled_dequant_##SUF(int nbits, int group, const void* packed, const void* scales, const void* zeros,   \
                                 int64_t N, int64_t K, void* out, int32_t out_dtype, int64_t ldo, hipStream_t st);  \
  void uintx_tiled_err_##SUF(int nbits, int group, const void* W, int64_t N, int64_t K, int64_t ldw,                \
                             const void* packed, const void* scales, const void* zeros, double* part, hipStream_t st); \
  void uintx_tiled_gemv_##SUF(int nbits, int group, int B, const void* packed, const void* scales, const void* zeros, \
                              int64_t N, int64_t K, const void* x, int64_t ldx, GemvOut out, hipStream_t st);
GWB_UINTX_TILED_DT(bf16)
GWB_UINTX_TILED_DT(f16)
GWB_UINTX_TILED_DT(f32)
#undef GWB_UINTX_TILED_DT
void launch_uintx_err_flat(int nbits, int32_t dt, int group, const void* W, int64_t N, int64_t K, int64_t ldw,
                           const void* packed, const void* scales, const void* zeros, double* part, hipStream_t st);

// ---- error finalize (common.hip): part[2*nblocks] -> out[3] = {sum w^2, sum e^2, dB}
void launch_err_finalize(const double* part, unsigned nblocks, double* out, hipStream_t st);

// ---- AWQ (awq.hip)
// Workspace bytes for a search over `rows` subsample rows of K columns (fixed by the
// shape alone); launch_awq carves it into the scaling powers, their log sums, the
// reciprocal tables and the per-block error partials.
size_t awq_workspace_bytes(int64_t rows, int64_t K, int n_alpha);
void launch_awq(const void* W, int32_t w_dtype, int64_t rows, int64_t row_step, int64_t K,
                int64_t ldw, const float* a, const double* alphas, int n_alpha, float* s_table,
                double* err, int32_t* best, void* workspace, hipStream_t st);

// ---- AWQ fold + MXFP4 requantize (fold.hip): column step, then row step, each
// rounded to bf16; outputs optional (NULL pointer = not written).
constexpr int kFoldNone = 0, kFoldMul = 1, kFoldDiv = 2;
void launch_fold(int col_op, int row_op, const void* W, int64_t N, int64_t K, int64_t ldw,
                 const float* col, const float* row, void* out, int64_t ldo, void* packed, void* e8m0,
                 hipStream_t st);

// ---- decode GEMV on quantized weights (gemv.hip); B <= 8 activation rows (bf16)
int gptq_gemv_splits(int64_t N, int64_t K);   // K splits; with more than one, part holds splits * B * N floats
void launch_gptq_gemv(bool sym, int group, int B, const void* qweight, const void* scales, const void* qzeros,
                      int64_t N, int64_t K, const void* x, int64_t ldx, void* y, int32_t y_dtype, int64_t ldy,
                      float* part, hipStream_t st);
// act-order GPTQ (group of channel k = g_idx[k]; K/G <= kActMaxGroups)
int gptq_act_gemv_splits(int64_t N, int64_t K);
void launch_gptq_act_gemv(bool sym, int group, int B, const void* qweight, const void* scales, const void* qzeros,
                          const int32_t* g_idx, int64_t N, int64_t K, const void* x, int64_t ldx, void* y,
                          int32_t y_dtype, int64_t ldy, float* part, hipStream_t st);
int mxfp4_gemv_splits(int64_t K, int B);      // K splits of the matrix-core GEMV (B >= 2); part as for GPTQ
void launch_mxfp4_gemv(int B, const void* packed, const void* e8m0, int64_t N, int64_t K, const void* x,
                       int64_t ldx, void* y, int32_t y_dtype, int64_t ldy, float* part, hipStream_t st);
// ---- prefill GEMM on quantized weights (gemm.hip): M activation rows (bf16), matrix
// cores; N % 8 == 0, K % 128 == 0. Workspace: GPTQ's group sums of x, then (small M)
// the K-split partial sums.
constexpr int kGemmMaxRows = 1 << 24;
// Decode batches on bf16-weight uintx in the tiled layout (N % 8 == 0, K % 512 == 0):
// the matrix-core path of gwb_gemv; float32 K-split partials in the workspace.
size_t uintx_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
int uintx_decode_splits(int nbits, int64_t B, int64_t N, int64_t K);
size_t uintx_decode_workspace_bytes(int nbits, int64_t B, int64_t N, int64_t K);
void launch_uintx_decode(int nbits, int group, const void* packed, const void* scales, const void* zeros, int64_t N,
                         int64_t K, const void* x, int64_t B, int64_t ldx, void* y, int32_t y_dtype, int64_t ldy,
                         void* workspace, hipStream_t st);
void launch_uintx_gemm(int nbits, int group, const void* packed, const void* scales, const void* zeros, int64_t N,
                       int64_t K, const void* x, int64_t M, int64_t ldx, void* y, int32_t y_dtype, int64_t ldy,
                       void* workspace, hipStream_t st);
size_t gemm_workspace_bytes(bool gptq, int group, int64_t M, int64_t N, int64_t K);
void launch_gptq_gemm(bool sym, int group, const void* qweight, const void* scales, const void* qzeros, int64_t N,
                      int64_t K, const void* x, int64_t M, int64_t ldx, void* y, int32_t y_dtype, int64_t ldy,
                      void* workspace, hipStream_t st);
void launch_mxfp4_gemm(const void* packed, const void* e8m0, int64_t N, int64_t K, const void* x, int64_t M,
                       int64_t ldx, void* y, int32_t y_dtype, int64_t ldy, void* workspace, hipStream_t st);
// uintx (uintx.hip): N % 8 == 0 and K % 512 == 0; with more than one split, part holds
// splits * B * N floats
bool uintx_gemv_supported(int64_t N, int64_t K);
int uintx_gemv_splits(int64_t K, int B);
void launch_uintx_gemv(int nbits, int32_t dt, int group, int B, const void* packed, const void* scales,
                       const void* zeros, int64_t N, int64_t K, const void* x, int64_t ldx, void* y, int32_t y_dtype,
                       int64_t ldy, float* part, hipStream_t st);
// y[b, n] = sum over s < S of part[(s * B + b) * N + n], in order
void launch_gemv_finalize(const float* part, int S, int B, int64_t N, void* y, int32_t y_dtype, int64_t ldy,
                          hipStream_t st);

// ---- measurement copy (common.hip)
void launch_stream_bench(int pattern, bool strided, unsigned blocks, void* dst, const void* src, uint64_t units,
                         hipStream_t st);

}  // namespace gwb
