/*
 * gwb.h — group-wise low-bit weight quantization on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libgwb.so. A linear layer's weight W is [N, K] (N output rows, K input
 * channels, K contiguous within a row, row stride ldw elements). Groups run along K.
 * Three formats, as the source pages define them:
 *
 *   GWB_GPTQ_SYM   page export_gptq_cpu.py, quantize_sym and the module docstring's
 *                  uint4b8 convention: w = (code - 8) * scale, code in [0, 15].
 *   GWB_GPTQ_ASYM  same page, quantize_asym: w = (code - zp) * scale, zp stored as is.
 *   GWB_MXFP4      page quantize_dflash_mxfp4.py, quantize_mxfp4 / dequantize_mxfp4:
 *                  e2m1 codes (round half to even), an E8M0 exponent per 32 weights.
 *   GWB_UINTX      page uintx_quant.py, UIntXQuantizer: affine uint2..uint7 with
 *                  preserve_zero, arithmetic in the weight's dtype (usually bfloat16),
 *                  planar power-of-two shards.
 *   GWB_MXFP4_PAGE_TIES  MXFP4 with the tie rule of the page's code instead of its
 *                  stated round-half-to-even: the first tied index, rounded down to even
 *                  (|x| / 2^e = 0.75, 1.75, 3.5 give 0, 1, 2 rather than 1, 2, 4). Same
 *                  stored layout; dequantization, SNR and the GEMV are MXFP4's.
 *   GWB_GPTQ_SYM_ACT / GWB_GPTQ_ASYM_ACT  GPTQ with act-order groups (the page stores
 *                  g_idx and writes desc_act into its checkpoint config): the groups are
 *                  the input channels taken in a caller-given order, G at a time; qweight
 *                  stays in channel order and g_idx[k] names channel k's group. Per-group
 *                  formulas as GWB_GPTQ_SYM / _ASYM; stored layout as GPTQ plus g_idx,
 *                  which gwb_quantize_act_order writes and dequantization and SNR read.
 *   GWB_GPTQ_SYM_GROUPED / GWB_GPTQ_ASYM_GROUPED  the same weight in group order, for the
 *                  decode GEMV (gwb_gptq_group_order makes it once): the channels taken
 *                  group by group, ascending inside a group, so group g sits at positions
 *                  g*G .. g*G + G - 1 and GPTQ's index-order layout applies; g_idx holds the
 *                  permutation (the channel at each position). Read by gwb_gemv only.
 *
 * Conventions for every entry point:
 *   - Pointers named d_* and every tensor pointer are DEVICE pointers owned by the
 *     caller (for example torch tensors). The library never allocates or frees device
 *     memory; buffers it needs beyond inputs and outputs come in as `workspace`.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *     asynchronously; nothing synchronizes except where stated.
 *   - Arguments are validated before anything is enqueued. On a non-zero return no
 *     kernel was launched and no output was written; gwb_last_error() describes why.
 *   - Empty shapes (N == 0 or K == 0) are valid and enqueue nothing.
 */
#ifndef GWB_H
#define GWB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GWB_OK = 0,
  GWB_E_ARG = -1,          /* NULL where a pointer is required, unknown enum, negative size */
  GWB_E_SHAPE = -2,        /* shape not divisible as the format requires */
  GWB_E_UNSUPPORTED = -3,  /* refused, as the pages refuse it (uintx nbits 8) or not provided */
  GWB_E_SIZE = -4,         /* a caller-declared buffer size is too small */
  GWB_E_HIP = -5           /* a HIP launch failed; gwb_last_error() names it */
} gwb_status;

typedef enum {
  GWB_GPTQ_SYM = 1, GWB_GPTQ_ASYM = 2, GWB_MXFP4 = 3, GWB_UINTX = 4, GWB_MXFP4_PAGE_TIES = 5,
  GWB_GPTQ_SYM_ACT = 6, GWB_GPTQ_ASYM_ACT = 7, GWB_GPTQ_SYM_GROUPED = 8, GWB_GPTQ_ASYM_GROUPED = 9
} gwb_format;
typedef enum { GWB_F32 = 0, GWB_BF16 = 1, GWB_F16 = 2 } gwb_dtype;

/* What to quantize to.
 *   format  gwb_format
 *   nbits   4 for GPTQ and MXFP4; 2..7 for UINTX (8 is refused with GWB_E_UNSUPPORTED:
 *           page uintx_quant.py, can_quantize, always left uint8 layers unquantized)
 *   group   GPTQ: 32, 64 or 128 (page export_gptq_cpu.py, --group, default 128);
 *           MXFP4: 32 (the page's GROUP); UINTX: 32, 64 (UIntXQuantizer's default
 *           group_size) or 128
 *   w_dtype gwb_dtype of W. GPTQ and MXFP4: GWB_BF16 or GWB_F32 (the pages widen W to
 *           float32). UINTX: GWB_BF16, GWB_F16 or GWB_F32; page uintx_quant.py runs the
 *           arithmetic in the weight's dtype (every op one float32 op rounded to it,
 *           float32 ops for GWB_F32) and stores the scale as that dtype. GWB_BF16 with
 *           group 64 and N*K % 512 == 0 takes the tiled kernels, everything else a
 *           two-pass path with a workspace.                                        */
typedef struct {
  int32_t format;
  int32_t nbits;
  int32_t group;
  int32_t w_dtype;
} gwb_qspec;

/* The quantized tensors (device pointers), per format:
 *   GPTQ   codes  int32 qweight [K/8, N]: nibble i of word (r, n) = code(k = 8r+i, n)
 *          scales fp16 [K/G, N]: the float32 group scale rounded to fp16 (RNE)
 *          zeros  int32 qzeros [K/G, N/8]: nibble i of word (g, q) = zero point of
 *                 column 8q+i; symmetric: every nibble 7; asymmetric: zp itself
 *          g_idx  int32 [K] = k / G; optional on output (NULL skips), unused on input;
 *                 act-order GPTQ: the group of channel k, required (input to
 *                 dequantization and SNR, output of gwb_quantize_act_order);
 *                 group-ordered GPTQ: perm, the channel at position k (required)
 *   MXFP4  codes  uint8 [N, K/2]: byte = code(2i) | code(2i+1) << 4, code = e2m1
 *                 magnitude index | sign << 3
 *          scales uint8 e8m0 [N, K/32] = exponent + 127;  zeros, g_idx unused (NULL)
 *   UINTX  codes  uint8 flat: one planar shard per power of two present in nbits, in
 *                 the order 4, 2, 1 (bits [off, off+k) of a code in the k-bit shard,
 *                 off counted from 0); shard k has ceil(N*K / (8/k)) bytes; byte i of
 *                 shard k = OR_j field(code[j*L + i]) << (j*k), L = that byte count,
 *                 codes taken in row-major order, zero-padded
 *          scales [N, K/G] of w_dtype (the bytes of its values, little-endian)
 *          zeros  uint8 [N, K/G] zero points in [0, 2**nbits - 1]; g_idx unused     */
typedef struct {
  void* codes;
  void* scales;
  void* zeros;
  void* g_idx;
} gwb_qtensors;

/* Byte sizes of the quantized tensors and of the workspace that gwb_quantize,
 * gwb_dequantize and gwb_snr need for (spec, N, K). */
typedef struct {
  size_t codes;
  size_t scales;
  size_t zeros;
  size_t g_idx;
  size_t workspace;
} gwb_sizes;

/* Validate (spec, N, K) and report buffer sizes. Host only, launches nothing.
 * Returns GWB_E_ARG / GWB_E_SHAPE / GWB_E_UNSUPPORTED as the format requires:
 *   GPTQ: K % group == 0, N % 8 == 0 (qzeros pack 8 columns per word); act-order
 *         GPTQ also K / group <= 256 and K * element size <= 64 KB (GWB_E_UNSUPPORTED);
 *   MXFP4: K % 32 == 0 (page quantize_mxfp4 asserts it);
 *   UINTX: K % group == 0 (can_quantize refuses otherwise).
 * Size: N * K < 2^31 elements (GWB_E_UNSUPPORTED beyond). MXFP4 rows are independent:
 * this query, gwb_quantize, gwb_quantize_snr (and its static variant), gwb_dequantize and
 * gwb_snr take MXFP4 up to N * K < 2^37 and run row bands of fewer than 2^31 elements
 * (the SNR partials of every band summed by one finalize); the GEMV, GEMM and fold keep
 * 2^31.                                                                          */
int gwb_query_sizes(const gwb_qspec* spec, int64_t N, int64_t K, gwb_sizes* out);

/* Quantize and pack W [N, K] (row stride ldw >= K elements, of spec->w_dtype).
 * Steps: per-group reduction (GPTQ sym amax, asym min/max, MXFP4 amax, UINTX
 * min/max extended to 0), scale and zero-point selection, round-and-clamp to codes,
 * bit packing; page export_gptq_cpu.py quantize_sym / quantize_asym / pack_int32,
 * page quantize_dflash_mxfp4.py quantize_mxfp4, page uintx_quant.py _quantize_impl /
 * pack_uintx. Every code, zero point, E8M0 byte and stored scale is bit-exact with
 * the step list of those passages (round half to even everywhere).
 * workspace/workspace_bytes: at least gwb_sizes.workspace bytes (may be NULL if 0). */
int gwb_quantize(const gwb_qspec* spec, const void* W, int64_t N, int64_t K, int64_t ldw,
                 const gwb_qtensors* out, void* workspace, size_t workspace_bytes,
                 void* stream);

/* Act-order GPTQ quantize (spec->format GWB_GPTQ_SYM_ACT or GWB_GPTQ_ASYM_ACT): group g is
 * the channels perm[g*G .. g*G + G - 1], quantized with page export_gptq_cpu.py's
 * quantize_sym / quantize_asym formulas; out->codes (qweight, channel order), scales and
 * zeros as for GPTQ, out->g_idx (required) int32 [K] with g_idx[perm[j]] = j / G.
 *   perm      device int32 [K], 16-byte aligned, a permutation of 0..K-1 (e.g. channels
 *             by decreasing activation magnitude); other contents give unspecified
 *             results, never an access outside the buffers
 *   workspace at least gwb_sizes.workspace bytes, 16-byte aligned (the float32 scale and
 *             zero point of every row and group)
 * gwb_quantize refuses these formats with GWB_E_ARG. */
int gwb_quantize_act_order(const gwb_qspec* spec, const void* W, int64_t N, int64_t K, int64_t ldw,
                           const int32_t* perm, const gwb_qtensors* out, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Act-order GPTQ into group order, once per weight, for the decode GEMV (GPTQ runtimes
 * reorder act-order weights at load time for the same reason): page export_gptq_cpu.py's
 * g_idx names each channel's group, so taking the channels group by group (ascending
 * inside a group) puts group g at positions g*G .. g*G + G - 1, where the index-order
 * GPTQ kernels read it with the activations gathered the same way.
 *   spec      GWB_GPTQ_SYM_ACT or GWB_GPTQ_ASYM_ACT (group 32, 64, 128; K/G <= 256)
 *   w         act-order tensors: codes (qweight [K/8, N], channel order) and g_idx [K]
 *             are read; scales and zeros are not touched (they stay valid as they are)
 *   codes_out int32 [K/8, N]: nibble i of word (r, n) = code of channel perm[8r + i]
 *   perm_out  int32 [K]: the channel at each position
 *   d_status  one device int32, written by the kernels: 0, or 1 when a group does not hold
 *             exactly G channels, 2 when a g_idx entry lies outside [0, K/G); on 1 or 2
 *             codes_out and perm_out are unspecified (every access stayed in bounds)
 * With spec->format changed to GWB_GPTQ_SYM_GROUPED / _ASYM_GROUPED, {codes_out, scales,
 * zeros, perm_out} is a valid gwb_qtensors for gwb_gemv. codes_out must not alias
 * w->codes. Empty shapes enqueue nothing (d_status is not written). */
int gwb_gptq_group_order(const gwb_qspec* spec, const gwb_qtensors* w, int64_t N, int64_t K, void* codes_out,
                         int32_t* perm_out, int32_t* d_status, void* stream);

/* Unpack and dequantize into out [N, K] (row stride ldo >= K) of out_dtype, in the
 * weight's own [N, K] layout for every format (the GPTQ transpose is undone).
 * GPTQ: (code - 8) * scale or (code - zp) * scale with the fp16 scale widened;
 * MXFP4: +-E2M1[code & 7] * 2**(e8m0 - 127); UINTX: r(r(q - zp) * scale), r the
 * rounding to w_dtype;
 * page export_gptq_cpu.py (module docstring), page quantize_dflash_mxfp4.py
 * dequantize_mxfp4, page uintx_quant.py _dequantize_native. Each value is the
 * correctly rounded result of an exact product, so bf16 and f32 outputs are exact
 * roundings. out_dtype: GWB_F32 or GWB_BF16; UINTX: GWB_F32 or w_dtype (its values
 * are of the weight dtype), anything else GWB_E_UNSUPPORTED. workspace as for
 * gwb_quantize. */
int gwb_dequantize(const gwb_qspec* spec, const gwb_qtensors* in, int64_t N, int64_t K,
                   void* out, int32_t out_dtype, int64_t ldo, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Reconstruction SNR of stored tensors against W, fused (the dequantized matrix is
 * never written). d_out (device, 3 doubles) receives
 *   d_out[0] = sum w**2, d_out[1] = sum (w - d)**2 (w - d a float32 subtraction, sums
 *   in float64), d_out[2] = 10 log10(d_out[0] / max(d_out[1], 1e-24)) dB,
 * which is page export_gptq_cpu.py's 20 log10(||w|| / max(||w - deq||, 1e-12)) and
 * gives page quantize_dflash_mxfp4.py's relative error 10**(-dB/20).
 * w is W as float32; d is the dequantized value in float32 (UINTX: the value of the
 * weight dtype that gwb_dequantize returns).
 * workspace: at least gwb_sizes.workspace bytes. Deterministic for a given shape.  */
int gwb_snr(const gwb_qspec* spec, const void* W, int64_t N, int64_t K, int64_t ldw,
            const gwb_qtensors* in, double* d_out, void* workspace, size_t workspace_bytes,
            void* stream);

/* Quantize and SNR in one call: what gwb_quantize followed by gwb_snr on the stored
 * tensors computes (page export_gptq_cpu.py computes its SNR inside its quantize
 * functions; here it is the SNR of the stored values, as gwb_snr defines it), with the
 * sums formed by the quantize kernel from the weights it has loaded and the values it
 * stores, so W is read once: MXFP4 (both tie modes), GPTQ sym / asym (groups in index
 * order; up to 16384 tiles of 32 rows x 512 k, larger matrices take the two passes) and
 * uintx in the tiled layout. Other shapes run the two calls in turn. Act-order formats:
 * GWB_E_ARG (they quantize with gwb_quantize_act_order). Arguments as gwb_quantize plus
 * d_out (device, 3 doubles, as gwb_snr); workspace at least gwb_sizes.workspace bytes,
 * 16-byte aligned. The sums match gwb_snr's up to the float64 summation order (the
 * MXFP4 pass runs the error kernel's order). N or K of 0: GWB_E_SHAPE.              */
int gwb_quantize_snr(const gwb_qspec* spec, const void* W, int64_t N, int64_t K, int64_t ldw,
                     const gwb_qtensors* out, double* d_out, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Workspace bytes for gwb_awq_search_mxfp4 on an [N, K] weight. Host only. */
int gwb_awq_workspace(int64_t N, int64_t K, int32_t n_alpha, int64_t max_rows, size_t* bytes);

/* AWQ-style alpha search on MXFP4, page quantize_dflash_mxfp4.py, search_scale, with
 * the diagonal surrogate objective of its module docstring.
 *   W        [N, K] of w_dtype, row stride ldw; rows W[::max(1, N / max_rows)][:max_rows]
 *            are used (max_rows > 0; the page uses 2048)
 *   d_a      float32 [K] per-input-channel mean |x| (device)
 *   alphas   HOST array of n_alpha doubles (1 <= n_alpha <= 16), e.g. 0, 0.1, ..., 1;
 *            NULL: d_s_table already holds the n_alpha scaling rows and is only read
 * Steps: a' = max(a, 1e-8); an = a' / mean(a'); per alpha s = clamp(an**alpha, 1e-2,
 * 1e2) / geomean (float64, rounded once to float32, written to d_s_table [n_alpha, K]);
 * X = W * s; D = dequant(quant_mxfp4(X)); err = sum(((D / s - W) * a')**2) with float32
 * elementwise ops and a float64 sum -> d_err [n_alpha] (device doubles);
 * d_best[0] = the first index with the strictly smallest error (device int32).
 * K % 32 == 0 is required; d_a, d_s_table and workspace must be 16-byte aligned, with
 * at least gwb_awq_workspace bytes of workspace. Deterministic for a given shape.    */
int gwb_awq_search_mxfp4(const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw,
                         const float* d_a, const double* alphas, int32_t n_alpha,
                         int64_t max_rows, float* d_s_table, double* d_err, int32_t* d_best,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Folding the AWQ scales into a bf16 weight, then requantizing it to MXFP4 (page
 * quantize_dflash_mxfp4.py, main and its module docstring: norm weights / s, the
 * columns of the projections that read the normed input * s, up's rows / down's s,
 * each rounded to bfloat16, then quantize_mxfp4 of every served linear).
 *   W        bf16 [N, K], row stride ldw (elements, multiple of 8), 16-byte aligned
 *   fold     column step (col_op with col: device float32 [K], 16-byte aligned) then
 *            row step (row_op with row: device float32 [N]); each op GWB_FOLD_NONE,
 *            GWB_FOLD_MUL or GWB_FOLD_DIV (IEEE), each result rounded to bfloat16
 *            (RNE); fold == NULL: no steps
 *   out_bf16 device bf16 [N, K] with row stride ldo (multiple of 8), or NULL
 *   mx       MXFP4 output as in gwb_quantize (codes = packed [N, K/2], scales =
 *            e8m0 [N, K/32]), or NULL / codes NULL for no quantization
 * At least one output is required. K % 32 == 0 with MXFP4 output, K % 8 == 0 without.
 * Only bf16 weights (E_UNSUPPORTED otherwise). Asynchronous on `stream`.            */
typedef enum { GWB_FOLD_NONE = 0, GWB_FOLD_MUL = 1, GWB_FOLD_DIV = 2 } gwb_fold_op;
typedef struct {
  const float* col;
  const float* row;
  int32_t col_op, row_op;
} gwb_fold;
int gwb_fold_mxfp4(const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw, const gwb_fold* fold,
                   void* out_bf16, int64_t ldo, const gwb_qtensors* mx, void* stream);

/* Decode GEMV on quantized weights: y[b, n] = sum_k x[b, k] * dequant(W)[n, k], the
 * weights read in their packed form. Page export_gptq_cpu.py: vLLM's W4A16 kernel
 * consumes the GPTQ tensors as stored (its lm_head note: the 131072 x 2048 head is the
 * largest read of a decode step); page quantize_dflash_mxfp4.py serves its linears as
 * MXFP4.
 *   spec, w  a GPTQ (sym or asym), MXFP4 or uintx weight as gwb_quantize wrote it, [N, K];
 *            uintx (page uintx_quant.py, forward: x times the dequantized weight of the
 *            weight dtype, r((q - zp) * s), converted to bf16 when it is not bf16) needs
 *            N % 8 == 0 and K % 512 == 0 (else GWB_E_UNSUPPORTED); act-order GPTQ reads
 *            w->g_idx (required); group-ordered GPTQ (gwb_gptq_group_order) reads its
 *            permutation in w->g_idx and runs as index-order GPTQ on the activations
 *            gathered into the workspace
 *   x        device bf16 [B, K], row stride ldx (multiple of 8), 16-byte aligned; 1 <= B <= 8
 *   y        device [B, N] of y_dtype (GWB_F32 or GWB_BF16, RNE), row stride ldy
 *   workspace at least gwb_gemv_workspace bytes (K-split partial sums of either path,
 *            the tile path's group sums, group order's gathered activations; none for
 *            MXFP4 below 5 rows of K <= 8192)
 * Paths: GPTQ with groups in index order (or group order) at B >= 2 runs gwb_gemm's
 * matrix-core tiles (and its numerics) when N % 8 == 0, K % 128 == 0, y and its rows
 * are 16-byte aligned (ldy % 8 == 0) and codes and scales are 16-byte aligned, as does
 * bf16-weight uintx at B >= 5 on weights of N >= 65536 rows (16-byte aligned codes);
 * MXFP4 at B >= 5 runs the GEMV's own matrix-core kernel (v_mfma_f32_16x16x32_bf16,
 * exact bf16 weights, the matrix cores' float32 sums); every other call runs the GEMV
 * kernels: products of dequantized values and activations exact in float32, float32
 * sums in a fixed order. All are deterministic for a given shape and path; the error is
 * bounded by the float32 accumulation.                                             */
int gwb_gemv_workspace(const gwb_qspec* spec, int64_t N, int64_t K, int64_t B, size_t* bytes);
int gwb_gemv(const gwb_qspec* spec, const gwb_qtensors* w, int64_t N, int64_t K, const void* x, int64_t B,
             int64_t ldx, void* y, int32_t y_dtype, int64_t ldy, void* workspace, size_t workspace_bytes,
             void* stream);

/* Prefill GEMM on quantized weights: y[m, n] = sum_k x[m, k] * dequant(W)[n, k] for M
 * rows of activations, the consumer of the stored tensors at prefill and batch sizes
 * (page export_gptq_cpu.py: vLLM's W4A16 kernels read the GPTQ tensors as written;
 * page quantize_dflash_mxfp4.py serves its linears as MXFP4). The weights are
 * dequantized on chip and multiplied on the matrix cores (bf16 operands, float32
 * accumulation).
 *   spec, w  GPTQ sym or asym (groups 32, 64, 128 in index order, or act-order groups
 *            in group order from gwb_gptq_group_order: the rows of x are gathered by its
 *            permutation into the workspace first), MXFP4, or uintx of bf16 weights
 *            (page uintx_quant.py, forward; K % 512 == 0), as gwb_quantize wrote it,
 *            [N, K]; N % 8 == 0 and K % 128 == 0 (else GWB_E_UNSUPPORTED); codes and
 *            scales 16-byte aligned
 *   x        device bf16 [M, K], row stride ldx (multiple of 8), 16-byte aligned;
 *            0 <= M <= 2^24 and M * ldx < 2^31
 *   y        device [M, N] of y_dtype (GWB_F32 or GWB_BF16, RNE), row stride ldy
 *            (multiple of 8), 16-byte aligned
 *   workspace at least gwb_gemm_workspace bytes: GPTQ the float32 group sums of x
 *            (K/G x M rounded up to 128, padded to 256 bytes); for M <= 64 with few
 *            column tiles also the float32 partial sums of a K split (splits x M x N),
 *            which a second kernel adds in split order; MXFP4 and uintx only the latter;
 *            group order first the gathered x (M x K bf16, padded to 256 bytes)
 * MXFP4 weights are exact bf16 operands, so every product is exact and only the
 * float32 sums round; so are uintx's forward weights bf16((q - zp) * s) (one rounding
 * of an exact product). uintx runs 16-row tiles that convert each weight once per 16
 * rows of x: a decode-batch kernel, slow for large M. GPTQ feeds the exact integers 128 + c and applies each group's
 * scale and zero point to the group's float32 sum: s * (sum x (128 + c) - (128 + z) *
 * sum x), the group sum of x taken in float64 and rounded once; the offset costs about
 * log2(143 / |c - z|) bits of the float32 sums relative to a direct sum. Deterministic
 * for a given shape. Returns GWB_OK without launching when M or N is 0.            */
int gwb_gemm_workspace(const gwb_qspec* spec, int64_t N, int64_t K, int64_t M, size_t* bytes);
int gwb_gemm(const gwb_qspec* spec, const gwb_qtensors* w, int64_t N, int64_t K, const void* x, int64_t M,
             int64_t ldx, void* y, int32_t y_dtype, int64_t ldy, void* workspace, size_t workspace_bytes,
             void* stream);

/* The AWQ scaling table on the host (page quantize_dflash_mxfp4.py, search_scale: the
 * per-alpha s of the search). a: HOST float32 [K] per-channel mean |x|; alphas: HOST
 * array of n_alpha doubles (1..16); s_out: HOST float32 [n_alpha, K]. Steps as in
 * gwb_awq_search_mxfp4 (float64, one rounding to float32); the device table agrees to
 * within one float32 ulp (float64 summation order). Touches no device memory.      */
int gwb_awq_scales_host(const float* a, int64_t K, const double* alphas, int32_t n_alpha, float* s_out);

/* gwb_quantize_snr for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. It takes no
 * workspace: the scratch it needs (the fused pass's per-block partial sums, or the
 * two-call fallback's code buffer) lives in a static device array of
 * GWB_STATIC_SCRATCH_BYTES that each device holds until the process ends. Arguments,
 * results and errors as gwb_quantize_snr; a shape whose gwb_sizes.workspace exceeds
 * GWB_STATIC_SCRATCH_BYTES returns GWB_E_SIZE (nothing enqueued). It allocates nothing.
 * All calls on one device share that device's array: calls that overlap on one GPU
 * (concurrent streams, other host threads) race and must be serialized by the caller. */
#define GWB_STATIC_SCRATCH_BYTES 262144
int gwb_quantize_snr_static(const gwb_qspec* spec, const void* W, int64_t N, int64_t K, int64_t ldw,
                            const gwb_qtensors* out, double* d_out, void* stream);

/* Measurement helper, not part of the method: a same-run streaming ceiling. Eight
 * 16-byte units in flight per lane, non-temporal loads of the larger side and non-temporal
 * 16-byte stores, in one of four patterns (`bytes` is the larger side):
 *   0 copy: read `bytes` from d_src, write `bytes` to d_dst;
 *   1 read: read `bytes` from d_src, write blocks * 1024 bytes (one word per thread) to d_dst;
 *   2 quantize-shaped: read `bytes` from d_src in 16-byte units, write 4 bytes per unit;
 *   3 dequantize-shaped: read 4 bytes per 16-byte unit written, `bytes` written.
 * OR-ing GWB_STREAM_STRIDED into the pattern makes the grid stride over the data; without
 * it each block streams one contiguous range. Both buffers must hold `bytes` (a multiple
 * of 64), 16-byte aligned; blocks in 1..65536 (pattern 1: blocks * 1024 <= bytes).
 * Asynchronous on `stream`. Returns GWB_E_ARG, GWB_E_UNSUPPORTED or GWB_E_SIZE (nothing
 * launched) on bad arguments. */
#define GWB_STREAM_STRIDED 4
int gwb_stream_bench(int32_t pattern, int32_t blocks, void* d_dst, const void* d_src, size_t bytes, void* stream);

/* Message for the last non-zero return on this thread ("" if none). */
const char* gwb_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GWB_H */
