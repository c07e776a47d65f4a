// C ABI of libgwb: argument validation, buffer sizes, launch selection. Declared in
// include/gwb.h. Everything is validated before the first launch, so a non-zero return
// means nothing was enqueued.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>
#include <cmath>

#include "gwb.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return GWB_OK;
}

int hip_check(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GWB_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Kernels index elements with 32-bit unsigned integers.
constexpr int64_t kMaxElems = (int64_t)1 << 31;
// MXFP4 rows are independent, so gwb_query_sizes, gwb_quantize, gwb_quantize_snr,
// gwb_dequantize and gwb_snr take MXFP4 shapes of up to kMaxBandedElems elements and run
// them as row bands of fewer than kMaxElems, each on offset pointers (the SNR partials of
// every band go to one finalize).
constexpr int64_t kMaxBandedElems = (int64_t)1 << 37;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// the two MXFP4 formats share every stored layout; only quantization differs
bool is_mxfp4(int32_t f) { return f == GWB_MXFP4 || f == GWB_MXFP4_PAGE_TIES; }
// act-order GPTQ shares GPTQ's stored layout; its groups come from g_idx
bool is_act(int32_t f) { return f == GWB_GPTQ_SYM_ACT || f == GWB_GPTQ_ASYM_ACT; }
// act-order GPTQ in group order (gwb_gptq_group_order): GPTQ's index-order layout, whose
// column j is channel g_idx[j] (there the channel permutation) of the layer
bool is_grouped(int32_t f) { return f == GWB_GPTQ_SYM_GROUPED || f == GWB_GPTQ_ASYM_GROUPED; }
bool is_gptq_sym(int32_t f) { return f == GWB_GPTQ_SYM || f == GWB_GPTQ_SYM_ACT || f == GWB_GPTQ_SYM_GROUPED; }
int refuse_grouped(const gwb_qspec* sp) {
  return is_grouped(sp->format)
             ? fail(GWB_E_UNSUPPORTED, "group-ordered GPTQ is made by gwb_gptq_group_order and read by gwb_gemv")
             : GWB_OK;
}

size_t elem_size(int32_t dt) { return dt == GWB_F32 ? 4 : 2; }

// banded: the call runs MXFP4 in row bands (see kMaxBandedElems).
int check_spec(const gwb_qspec* sp, int64_t N, int64_t K, bool banded = false) {
  if (!sp) return fail(GWB_E_ARG, "spec is NULL");
  if (N < 0 || K < 0) return fail(GWB_E_ARG, "negative shape N=%lld K=%lld", (long long)N, (long long)K);
  if (sp->w_dtype != GWB_F32 && sp->w_dtype != GWB_BF16 && sp->w_dtype != GWB_F16)
    return fail(GWB_E_ARG, "unknown w_dtype %d", sp->w_dtype);
  if (sp->w_dtype == GWB_F16 && sp->format != GWB_UINTX)
    return fail(GWB_E_UNSUPPORTED, "float16 weights are provided for UINTX only");
  const bool bands = banded && is_mxfp4(sp->format);
  if (N > 0 && K > 0 && (N >= kMaxElems || K >= kMaxElems || N * K >= (bands ? kMaxBandedElems : kMaxElems)))
    return fail(GWB_E_UNSUPPORTED, "N*K = %lld exceeds %s elements", (long long)(N * K), bands ? "2^37" : "2^31");
  switch (sp->format) {
    case GWB_GPTQ_SYM:
    case GWB_GPTQ_ASYM:
    case GWB_GPTQ_SYM_ACT:
    case GWB_GPTQ_ASYM_ACT:
    case GWB_GPTQ_SYM_GROUPED:
    case GWB_GPTQ_ASYM_GROUPED:
      if (sp->nbits != 4) return fail(GWB_E_ARG, "GPTQ is 4-bit, got nbits=%d", sp->nbits);
      if (sp->group <= 0) return fail(GWB_E_ARG, "group must be positive, got %d", sp->group);
      if (sp->group != 32 && sp->group != 64 && sp->group != 128)
        return fail(GWB_E_UNSUPPORTED, "GPTQ group %d not provided (32, 64, 128)", sp->group);
      if (K % sp->group) return fail(GWB_E_SHAPE, "K=%lld not divisible by group %d", (long long)K, sp->group);
      if (N % 8) return fail(GWB_E_SHAPE, "GPTQ qzeros pack 8 columns per int32: N=%lld not divisible by 8",
                             (long long)N);
      if (is_act(sp->format) && K / sp->group > gwb::kActMaxGroups)
        return fail(GWB_E_UNSUPPORTED, "act-order GPTQ holds at most %d groups per row, got K/G=%lld",
                    gwb::kActMaxGroups, (long long)(K / sp->group));
      if (is_act(sp->format) && K * (int64_t)elem_size(sp->w_dtype) > gwb::kActMaxRowBytes)
        return fail(GWB_E_UNSUPPORTED, "act-order GPTQ holds a weight row of at most %lld bytes, got %lld",
                    (long long)gwb::kActMaxRowBytes, (long long)(K * (int64_t)elem_size(sp->w_dtype)));
      return GWB_OK;
    case GWB_MXFP4:
    case GWB_MXFP4_PAGE_TIES:
      if (sp->nbits != 4) return fail(GWB_E_ARG, "MXFP4 is 4-bit, got nbits=%d", sp->nbits);
      if (sp->group != 32) return fail(GWB_E_UNSUPPORTED, "MXFP4 blocks are 32 weights, got group %d", sp->group);
      if (K % 32) return fail(GWB_E_SHAPE, "K=%lld not divisible by 32", (long long)K);
      return GWB_OK;
    case GWB_UINTX:
      if (sp->nbits == 8)
        return fail(GWB_E_UNSUPPORTED, "uint8 is refused: it was always left unquantized");
      if (sp->nbits < 2 || sp->nbits > 8) return fail(GWB_E_ARG, "uintx nbits must be 2..7, got %d", sp->nbits);
      if (sp->group <= 0) return fail(GWB_E_ARG, "group must be positive, got %d", sp->group);
      if (sp->group != 32 && sp->group != 64 && sp->group != 128)
        return fail(GWB_E_UNSUPPORTED, "uintx group %d not provided (32, 64, 128)", sp->group);
      if (K % sp->group) return fail(GWB_E_SHAPE, "K=%lld not divisible by group %d", (long long)K, sp->group);
      return GWB_OK;
    default:
      return fail(GWB_E_ARG, "unknown format %d", sp->format);
  }
}

size_t uintx_packed_bytes(int nbits, int64_t numel) {
  size_t b = 0;
  if (nbits & 4) b += (size_t)((numel + 1) / 2);
  if (nbits & 2) b += (size_t)((numel + 3) / 4);
  if (nbits & 1) b += (size_t)((numel + 7) / 8);
  return b;
}

// Rows of an MXFP4 band: fewer than kMaxElems elements (all N when the shape is below).
int64_t mx_band_rows(int64_t N, int64_t K) {
  const int64_t r = (kMaxElems - 1) / (K > 0 ? K : 1);
  return r < N ? r : N;
}
// f(r0, n) for each band of rows [r0, r0 + n), in order.
template <typename F>
void mx_bands(int64_t N, int64_t K, F&& f) {
  const int64_t R = mx_band_rows(N, K);
  for (int64_t r0 = 0; r0 < N; r0 += R) f(r0, N - r0 < R ? N - r0 : R);
}
unsigned mx_err_blocks(int64_t N, int64_t K) {
  unsigned nb = 0;
  mx_bands(N, K, [&](int64_t, int64_t n) { nb += gwb::mxfp4_err_blocks(n, K); });
  return nb;
}

unsigned err_blocks(const gwb_qspec* sp, int64_t N, int64_t K) {
  switch (sp->format) {
    case GWB_MXFP4:
    case GWB_MXFP4_PAGE_TIES: return mx_err_blocks(N, K);
    case GWB_UINTX: return gwb::uintx_err_blocks(sp->w_dtype, sp->group, N, K);
    case GWB_GPTQ_SYM_ACT:
    case GWB_GPTQ_ASYM_ACT: return gwb::gptq_act_err_blocks(N, K);
    default: return gwb::gptq_err_blocks(sp->group, N, K);
  }
}

gwb_sizes sizes_of(const gwb_qspec* sp, int64_t N, int64_t K) {
  gwb_sizes s{};
  const int64_t G = sp->group;
  switch (sp->format) {
    case GWB_GPTQ_SYM:
    case GWB_GPTQ_ASYM:
    case GWB_GPTQ_SYM_ACT:
    case GWB_GPTQ_ASYM_ACT:
    case GWB_GPTQ_SYM_GROUPED:
    case GWB_GPTQ_ASYM_GROUPED:
      s.codes = (size_t)(K / 8 * N * 4);
      s.scales = (size_t)(K / G * N * 2);
      s.zeros = (size_t)(K / G * (N / 8) * 4);
      s.g_idx = (size_t)(K * 4);
      break;
    case GWB_MXFP4:
    case GWB_MXFP4_PAGE_TIES:
      s.codes = (size_t)(N * K / 2);
      s.scales = (size_t)(N * K / 32);
      break;
    default:
      s.codes = uintx_packed_bytes(sp->nbits, N * K);
      s.scales = (size_t)(N * (K / G)) * elem_size(sp->w_dtype);   // the weight dtype
      s.zeros = (size_t)(N * (K / G));
      break;
  }
  size_t ws = 0;
  if (N > 0 && K > 0 && !is_grouped(sp->format)) {
    ws = (size_t)err_blocks(sp, N, K) * 2 * sizeof(double);
    if (sp->format == GWB_UINTX) {
      size_t c = gwb::uintx_code_workspace(sp->w_dtype, sp->group, N, K);
      ws = c > ws ? c : ws;
    }
    if (is_act(sp->format)) {     // float32 scale and zero point of every (row, group)
      size_t c = gwb::gptq_act_workspace_bytes(N, K, sp->group);
      ws = c > ws ? c : ws;
    }
  }
  s.workspace = ws;
  return s;
}

int check_weight(const gwb_qspec* sp, const void* W, int64_t K, int64_t ldw) {
  if (!W) return fail(GWB_E_ARG, "W is NULL");
  if (ldw < K) return fail(GWB_E_ARG, "ldw=%lld < K=%lld", (long long)ldw, (long long)K);
  if (!aligned16(W) || ((size_t)ldw * elem_size(sp->w_dtype)) % 16)
    return fail(GWB_E_UNSUPPORTED, "W and its row stride must be 16-byte aligned");
  return GWB_OK;
}

int check_tensors(const gwb_qspec* sp, const gwb_qtensors* q) {
  if (!q) return fail(GWB_E_ARG, "tensors struct is NULL");
  if (!q->codes || !q->scales) return fail(GWB_E_ARG, "codes and scales are required");
  if (!is_mxfp4(sp->format) && !q->zeros) return fail(GWB_E_ARG, "zeros is required for this format");
  if (is_act(sp->format) && !q->g_idx) return fail(GWB_E_ARG, "act-order GPTQ needs g_idx");
  if (is_grouped(sp->format) && !q->g_idx) return fail(GWB_E_ARG, "group-ordered GPTQ needs its permutation in g_idx");
  if (!aligned16(q->codes) || !aligned16(q->scales) || (q->zeros && !aligned16(q->zeros)) ||
      ((is_act(sp->format) || is_grouped(sp->format)) && !aligned16(q->g_idx)))
    return fail(GWB_E_UNSUPPORTED, "quantized tensors must be 16-byte aligned");
  return GWB_OK;
}

}  // namespace

extern "C" {

const char* gwb_last_error(void) { return g_err.c_str(); }

int gwb_query_sizes(const gwb_qspec* spec, int64_t N, int64_t K, gwb_sizes* out) {
  if (int rc = check_spec(spec, N, K, true)) return rc;
  if (!out) return fail(GWB_E_ARG, "out is NULL");
  *out = sizes_of(spec, N, K);
  return ok();
}

int gwb_quantize(const gwb_qspec* spec, const void* W, int64_t N, int64_t K, int64_t ldw,
                 const gwb_qtensors* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (int rc = check_spec(spec, N, K, true)) return rc;
  if (is_act(spec->format))
    return fail(GWB_E_ARG, "act-order GPTQ takes the channel order: use gwb_quantize_act_order");
  if (int rc = refuse_grouped(spec)) return rc;
  if (N == 0 || K == 0) return ok();          // empty: valid, nothing to enqueue
  if (int rc = check_weight(spec, W, K, ldw)) return rc;
  if (int rc = check_tensors(spec, out)) return rc;
  if (spec->format == GWB_UINTX) {
    const size_t need = gwb::uintx_code_workspace(spec->w_dtype, spec->group, N, K);
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(GWB_E_SIZE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    if (need > 0 && !aligned16(workspace)) return fail(GWB_E_UNSUPPORTED, "workspace must be 16-byte aligned");
  }
  hipStream_t st = (hipStream_t)stream;
  switch (spec->format) {
    case GWB_GPTQ_SYM:
    case GWB_GPTQ_ASYM:
      gwb::launch_gptq_quant(spec->format == GWB_GPTQ_SYM, spec->group, W, spec->w_dtype, N, K, ldw, out->codes,
                             out->scales, out->zeros, out->g_idx, st);
      break;
    case GWB_MXFP4:
    case GWB_MXFP4_PAGE_TIES:
      mx_bands(N, K, [&](int64_t r0, int64_t n) {
        gwb::launch_mxfp4_quant(spec->format == GWB_MXFP4_PAGE_TIES,
                                (const char*)W + r0 * ldw * (int64_t)elem_size(spec->w_dtype), spec->w_dtype, n, K,
                                ldw, (uint8_t*)out->codes + r0 * (K / 2), (uint8_t*)out->scales + r0 * (K / 32),
                                nullptr, st);
      });
      break;
    default:
      gwb::launch_uintx_quant(spec->nbits, spec->w_dtype, spec->group, W, N, K, ldw, out->codes, out->scales,
                              out->zeros, workspace, nullptr, st);
  }
  return hip_check("quantize launch");
}

// Quantize and the reconstruction SNR of what was stored, in one pass over W where the
// quantize kernel can form the sums itself (MXFP4, GPTQ in index order while its tiles
// fit the partials, uintx in the tiled layout); otherwise the two calls in turn.
int gwb_quantize_snr(const gwb_qspec* spec, const void* W, int64_t N, int64_t K, int64_t ldw,
                     const gwb_qtensors* out, double* d_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (int rc = check_spec(spec, N, K, true)) return rc;
  if (is_act(spec->format)) return fail(GWB_E_ARG, "act-order GPTQ quantizes with gwb_quantize_act_order");
  if (int rc = refuse_grouped(spec)) return rc;
  if (!d_out) return fail(GWB_E_ARG, "d_out is NULL");
  if (N == 0 || K == 0) return fail(GWB_E_SHAPE, "SNR of an empty matrix is undefined");
  if (int rc = check_weight(spec, W, K, ldw)) return rc;
  if (int rc = check_tensors(spec, out)) return rc;
  bool fused = true;
  if (spec->format == GWB_GPTQ_SYM || spec->format == GWB_GPTQ_ASYM)
    fused = gwb::gptq_quant_snr_fits(spec->group, N, K);
  else if (spec->format == GWB_UINTX)
    fused = gwb::uintx_tiled(spec->w_dtype, spec->group, N, K);
  const unsigned nb = err_blocks(spec, N, K);
  size_t need = (size_t)nb * 2 * sizeof(double);
  if (!fused && spec->format == GWB_UINTX) {   // the two-pass quantize's code buffer shares the workspace
    const size_t c = gwb::uintx_code_workspace(spec->w_dtype, spec->group, N, K);
    need = c > need ? c : need;
  }
  // checked before anything is enqueued, the unfused pair of calls included
  if (!workspace || workspace_bytes < need)
    return fail(GWB_E_SIZE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!aligned16(workspace)) return fail(GWB_E_UNSUPPORTED, "workspace must be 16-byte aligned");
  if (!fused) {
    if (int rc = gwb_quantize(spec, W, N, K, ldw, out, workspace, workspace_bytes, stream)) return rc;
    return gwb_snr(spec, W, N, K, ldw, out, d_out, workspace, workspace_bytes, stream);
  }
  hipStream_t st = (hipStream_t)stream;
  double* part = (double*)workspace;
  if (spec->format == GWB_GPTQ_SYM || spec->format == GWB_GPTQ_ASYM)
    gwb::launch_gptq_quant_snr(spec->format == GWB_GPTQ_SYM, spec->group, W, spec->w_dtype, N, K, ldw, out->codes,
                               out->scales, out->zeros, out->g_idx, part, st);
  else if (is_mxfp4(spec->format)) {
    double* p = part;
    mx_bands(N, K, [&](int64_t r0, int64_t n) {
      gwb::launch_mxfp4_quant(spec->format == GWB_MXFP4_PAGE_TIES,
                              (const char*)W + r0 * ldw * (int64_t)elem_size(spec->w_dtype), spec->w_dtype, n, K, ldw,
                              (uint8_t*)out->codes + r0 * (K / 2), (uint8_t*)out->scales + r0 * (K / 32), p, st);
      p += 2 * (size_t)gwb::mxfp4_err_blocks(n, K);
    });
  } else
    gwb::launch_uintx_quant(spec->nbits, spec->w_dtype, spec->group, W, N, K, ldw, out->codes, out->scales,
                            out->zeros, nullptr, part, st);
  gwb::launch_err_finalize(part, nb, d_out, st);
  return hip_check("quantize_snr launch");
}

int gwb_dequantize(const gwb_qspec* spec, const gwb_qtensors* in, int64_t N, int64_t K, void* out,
                   int32_t out_dtype, int64_t ldo, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (int rc = check_spec(spec, N, K, true)) return rc;
  if (int rc = refuse_grouped(spec)) return rc;
  if (out_dtype != GWB_F32 && out_dtype != GWB_BF16 && out_dtype != GWB_F16)
    return fail(GWB_E_ARG, "unknown out_dtype %d", out_dtype);
  // UINTX values are of the weight dtype (float32 holds them exactly); the other
  // formats' exact products are rounded once to bf16 or kept in float32.
  if (spec->format == GWB_UINTX ? (out_dtype != GWB_F32 && out_dtype != spec->w_dtype) : out_dtype == GWB_F16)
    return fail(GWB_E_UNSUPPORTED, "out_dtype %d not provided for this format and weight dtype", out_dtype);
  if (N == 0 || K == 0) return ok();          // empty: valid, nothing to enqueue
  if (int rc = check_tensors(spec, in)) return rc;
  if (!out) return fail(GWB_E_ARG, "out is NULL");
  if (ldo < K) return fail(GWB_E_ARG, "ldo=%lld < K=%lld", (long long)ldo, (long long)K);
  if (!aligned16(out) || ((size_t)ldo * elem_size(out_dtype)) % 16)
    return fail(GWB_E_UNSUPPORTED, "out and its row stride must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  switch (spec->format) {
    case GWB_GPTQ_SYM:
    case GWB_GPTQ_ASYM:
      gwb::launch_gptq_dequant(spec->format == GWB_GPTQ_SYM, spec->group, in->codes, in->scales, in->zeros, N, K,
                               out, out_dtype, ldo, st);
      break;
    case GWB_GPTQ_SYM_ACT:
    case GWB_GPTQ_ASYM_ACT:
      gwb::launch_gptq_act_dequant(is_gptq_sym(spec->format), spec->group, in->codes, in->scales, in->zeros,
                                   (const int32_t*)in->g_idx, N, K, out, out_dtype, ldo, st);
      break;
    case GWB_MXFP4:
    case GWB_MXFP4_PAGE_TIES:
      mx_bands(N, K, [&](int64_t r0, int64_t n) {
        gwb::launch_mxfp4_dequant((const uint8_t*)in->codes + r0 * (K / 2), (const uint8_t*)in->scales + r0 * (K / 32),
                                  n, K, (char*)out + r0 * ldo * (int64_t)elem_size(out_dtype), out_dtype, ldo, st);
      });
      break;
    default:
      gwb::launch_uintx_dequant(spec->nbits, spec->w_dtype, spec->group, in->codes, in->scales, in->zeros, N, K,
                                out, out_dtype, ldo, st);
  }
  return hip_check("dequantize launch");
}

int gwb_snr(const gwb_qspec* spec, const void* W, int64_t N, int64_t K, int64_t ldw, const gwb_qtensors* in,
            double* d_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (int rc = check_spec(spec, N, K, true)) return rc;
  if (int rc = refuse_grouped(spec)) return rc;
  if (int rc = check_weight(spec, W, K, ldw)) return rc;
  if (int rc = check_tensors(spec, in)) return rc;
  if (!d_out) return fail(GWB_E_ARG, "d_out is NULL");
  if (N == 0 || K == 0) return fail(GWB_E_SHAPE, "SNR of an empty matrix is undefined");
  const unsigned nb = err_blocks(spec, N, K);
  const size_t need = (size_t)nb * 2 * sizeof(double);
  if (!workspace || workspace_bytes < need)
    return fail(GWB_E_SIZE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!aligned16(workspace)) return fail(GWB_E_UNSUPPORTED, "workspace must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  double* part = (double*)workspace;
  switch (spec->format) {
    case GWB_GPTQ_SYM:
    case GWB_GPTQ_ASYM:
      gwb::launch_gptq_err(spec->format == GWB_GPTQ_SYM, spec->group, W, spec->w_dtype, N, K, ldw, in->codes,
                           in->scales, in->zeros, part, st);
      break;
    case GWB_GPTQ_SYM_ACT:
    case GWB_GPTQ_ASYM_ACT:
      gwb::launch_gptq_act_err(is_gptq_sym(spec->format), spec->group, W, spec->w_dtype, N, K, ldw, in->codes,
                               in->scales, in->zeros, (const int32_t*)in->g_idx, part, st);
      break;
    case GWB_MXFP4:
    case GWB_MXFP4_PAGE_TIES: {
      double* p = part;
      mx_bands(N, K, [&](int64_t r0, int64_t n) {
        gwb::launch_mxfp4_err((const char*)W + r0 * ldw * (int64_t)elem_size(spec->w_dtype), spec->w_dtype, n, K, ldw,
                              (const uint8_t*)in->codes + r0 * (K / 2), (const uint8_t*)in->scales + r0 * (K / 32), p,
                              st);
        p += 2 * (size_t)gwb::mxfp4_err_blocks(n, K);
      });
      break;
    }
    default:
      gwb::launch_uintx_err(spec->nbits, spec->w_dtype, spec->group, W, N, K, ldw, in->codes, in->scales,
                            in->zeros, part, st);
  }
  gwb::launch_err_finalize(part, nb, d_out, st);
  return hip_check("snr launch");
}

int gwb_quantize_act_order(const gwb_qspec* spec, const void* W, int64_t N, int64_t K, int64_t ldw,
                           const int32_t* perm, const gwb_qtensors* out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (int rc = check_spec(spec, N, K)) return rc;
  if (!is_act(spec->format)) return fail(GWB_E_ARG, "format must be GWB_GPTQ_SYM_ACT or GWB_GPTQ_ASYM_ACT");
  if (N == 0 || K == 0) return ok();          // empty: valid, nothing to enqueue
  if (int rc = check_weight(spec, W, K, ldw)) return rc;
  if (int rc = check_tensors(spec, out)) return rc;
  if (!perm) return fail(GWB_E_ARG, "perm is NULL");
  if (!aligned16(perm)) return fail(GWB_E_UNSUPPORTED, "perm must be 16-byte aligned");
  const size_t need = gwb::gptq_act_workspace_bytes(N, K, spec->group);
  if (!workspace || workspace_bytes < need)
    return fail(GWB_E_SIZE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!aligned16(workspace)) return fail(GWB_E_UNSUPPORTED, "workspace must be 16-byte aligned");
  gwb::launch_gptq_act_quant(is_gptq_sym(spec->format), spec->group, W, spec->w_dtype, N, K, ldw, perm, out->codes,
                             out->scales, out->zeros, (int32_t*)out->g_idx, workspace, (hipStream_t)stream);
  return hip_check("act-order quantize launch");
}

int gwb_gptq_group_order(const gwb_qspec* spec, const gwb_qtensors* w, int64_t N, int64_t K, void* codes_out,
                         int32_t* perm_out, int32_t* d_status, void* stream) {
  if (int rc = check_spec(spec, N, K)) return rc;
  if (!is_act(spec->format)) return fail(GWB_E_ARG, "format must be GWB_GPTQ_SYM_ACT or GWB_GPTQ_ASYM_ACT");
  if (!w || !w->codes || !w->g_idx) return fail(GWB_E_ARG, "the act-order codes and g_idx are required");
  if (!codes_out || !perm_out || !d_status) return fail(GWB_E_ARG, "codes_out, perm_out and d_status are required");
  if (!aligned16(w->codes) || !aligned16(w->g_idx) || !aligned16(codes_out) || !aligned16(perm_out))
    return fail(GWB_E_UNSUPPORTED, "tensors must be 16-byte aligned");
  if (codes_out == w->codes) return fail(GWB_E_ARG, "codes_out must not be the input codes");
  if (N == 0 || K == 0) return ok();          // empty: valid, nothing to enqueue
  gwb::launch_gptq_group_order(spec->group, w->codes, (const int32_t*)w->g_idx, N, K, codes_out, perm_out, d_status,
                               (hipStream_t)stream);
  return hip_check("group order launch");
}

static int awq_rows(int64_t N, int64_t max_rows, int64_t* rows, int64_t* step) {
  *step = N / max_rows > 1 ? N / max_rows : 1;
  int64_t avail = (N + *step - 1) / *step;
  *rows = avail < max_rows ? avail : max_rows;
  return 0;
}

int gwb_awq_workspace(int64_t N, int64_t K, int32_t n_alpha, int64_t max_rows, size_t* bytes) {
  if (!bytes) return fail(GWB_E_ARG, "bytes is NULL");
  if (N <= 0 || K <= 0 || max_rows <= 0) return fail(GWB_E_ARG, "N, K and max_rows must be positive");
  if (n_alpha < 1 || n_alpha > 16) return fail(GWB_E_ARG, "n_alpha must be 1..16, got %d", n_alpha);
  int64_t rows, step;
  awq_rows(N, max_rows, &rows, &step);
  *bytes = gwb::awq_workspace_bytes(rows, K, n_alpha);
  return ok();
}

int gwb_awq_search_mxfp4(const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw, const float* d_a,
                         const double* alphas, int32_t n_alpha, int64_t max_rows, float* d_s_table, double* d_err,
                         int32_t* d_best, void* workspace, size_t workspace_bytes, void* stream) {
  gwb_qspec sp{GWB_MXFP4, 4, 32, w_dtype};
  if (N <= 0 || K <= 0) return fail(GWB_E_ARG, "N and K must be positive");
  if (int rc = check_spec(&sp, N, K)) return rc;
  if (int rc = check_weight(&sp, W, K, ldw)) return rc;
  if (!d_a || !d_s_table || !d_err || !d_best) return fail(GWB_E_ARG, "a, s_table, err and best are required");
  if (!aligned16(d_s_table) || !aligned16(d_a)) return fail(GWB_E_UNSUPPORTED, "a and s_table must be 16-byte aligned");
  if (n_alpha < 1 || n_alpha > 16) return fail(GWB_E_ARG, "n_alpha must be 1..16, got %d", n_alpha);
  if (max_rows <= 0) return fail(GWB_E_ARG, "max_rows must be positive");
  int64_t rows, step;
  awq_rows(N, max_rows, &rows, &step);
  const size_t need = gwb::awq_workspace_bytes(rows, K, n_alpha);
  if (!workspace || workspace_bytes < need)
    return fail(GWB_E_SIZE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!aligned16(workspace)) return fail(GWB_E_UNSUPPORTED, "workspace must be 16-byte aligned");
  gwb::launch_awq(W, w_dtype, rows, step, K, ldw, d_a, alphas, n_alpha, d_s_table, d_err, d_best,
                  workspace, (hipStream_t)stream);
  return hip_check("awq launch");
}

int gwb_fold_mxfp4(const void* W, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw, const gwb_fold* fold,
                   void* out_bf16, int64_t ldo, const gwb_qtensors* mx, void* stream) {
  if (w_dtype != GWB_BF16) return fail(GWB_E_UNSUPPORTED, "the fold takes bf16 weights (the pages' dtype)");
  if (N < 0 || K < 0) return fail(GWB_E_ARG, "negative shape N=%lld K=%lld", (long long)N, (long long)K);
  if (N > 0 && K > 0 && (N >= kMaxElems || K >= kMaxElems || N * K >= kMaxElems))
    return fail(GWB_E_UNSUPPORTED, "N*K = %lld exceeds 2^31 elements", (long long)(N * K));
  const gwb_fold none{nullptr, nullptr, GWB_FOLD_NONE, GWB_FOLD_NONE};
  const gwb_fold* f = fold ? fold : &none;
  for (int32_t op : {f->col_op, f->row_op})
    if (op != GWB_FOLD_NONE && op != GWB_FOLD_MUL && op != GWB_FOLD_DIV) return fail(GWB_E_ARG, "unknown fold op %d", op);
  const bool want_mx = mx && mx->codes;
  if (!out_bf16 && !want_mx) return fail(GWB_E_ARG, "nothing to write: out_bf16 and mx are both NULL");
  if (K % (want_mx ? 32 : 8)) return fail(GWB_E_SHAPE, "K=%lld must be a multiple of %d", (long long)K, want_mx ? 32 : 8);
  if (N == 0 || K == 0) return ok();
  if (!W) return fail(GWB_E_ARG, "W is NULL");
  if (ldw < K) return fail(GWB_E_ARG, "ldw=%lld < K=%lld", (long long)ldw, (long long)K);
  if (!aligned16(W) || ldw % 8) return fail(GWB_E_UNSUPPORTED, "W and its row stride must be 16-byte aligned");
  if (f->col_op != GWB_FOLD_NONE && (!f->col || !aligned16(f->col)))
    return fail(GWB_E_ARG, "the column step needs a 16-byte aligned col vector");
  if (f->row_op != GWB_FOLD_NONE && !f->row) return fail(GWB_E_ARG, "the row step needs a row vector");
  if (out_bf16 && (ldo < K || !aligned16(out_bf16) || ldo % 8))
    return fail(GWB_E_UNSUPPORTED, "out_bf16 needs ldo >= K and a 16-byte aligned start and row stride");
  if (want_mx && (!mx->scales || !aligned16(mx->codes)))
    return fail(GWB_E_ARG, "MXFP4 output needs 16-byte aligned codes and an e8m0 buffer");
  gwb::launch_fold(f->col_op, f->row_op, W, N, K, ldw, f->col, f->row, out_bf16, ldo, want_mx ? mx->codes : nullptr,
                   want_mx ? mx->scales : nullptr, (hipStream_t)stream);
  return hip_check("fold launch");
}

// Batches that the matrix-core tile kernels of gwb_gemm take faster than the GEMV
// kernels: GPTQ with groups in index order from 2 rows, when the shape fits the tile
// (N % 8 == 0, K % 128 == 0). MXFP4 batches stay with the GEMV, whose own matrix-core
// kernel takes 5 to 8 rows.
static bool gemv_shape_via_gemm(const gwb_qspec* sp, int64_t N, int64_t K, int64_t B) {
  if (N % 8 || K % 128 || B * K >= kMaxElems) return false;
  return (sp->format == GWB_GPTQ_SYM || sp->format == GWB_GPTQ_ASYM) && B >= 2;
}
// bf16-weight uintx batches go to the matrix-core decode kernel where it is faster than
// the GEMV kernels: from 2 rows for 2 and 4 bits (one plane per wavefront), from 3 rows
// for 3, 5 and 6 bits (two planes), from 5 rows for 7 bits (three planes: fewer
// wavefronts per SIMD). Measured on the 131072 x 2048 head, cold, decode against GEMV:
// B = 8, uintx4 42.5 against 62.5 us (the GEMM tiles), uintx7 78.5 against 88.6 (tiles);
// B = 3, uintx3 49.3 against 56.8; B = 2, uintx3 48.1 against 45.6, uintx7 74.6 against
// 61.6; B = 1, uintx4 38.6 against 34.8.
static bool gemm_uintx_shape(const gwb_qspec* sp, int64_t N, int64_t K) {
  return sp->format == GWB_UINTX && sp->w_dtype == GWB_BF16 && N % 8 == 0 && K % 512 == 0;
}
static bool gemv_uintx_via_decode(const gwb_qspec* sp, int64_t N, int64_t K, int64_t B) {
  if (!gemm_uintx_shape(sp, N, K) || B * K >= kMaxElems) return false;
  if (sp->nbits == 2 || sp->nbits == 4) return B >= 2;
  return B >= (sp->nbits == 7 ? 5 : 3);
}

// The GEMV kernels' K-split partial sums (none with a single split).
static size_t gemv_kernel_workspace(const gwb_qspec* sp, int64_t N, int64_t K, int64_t B) {
  int S = 0;
  if (sp->format == GWB_GPTQ_SYM || sp->format == GWB_GPTQ_ASYM) S = gwb::gptq_gemv_splits(N, K);
  if (is_act(sp->format)) S = gwb::gptq_act_gemv_splits(N, K);
  if (sp->format == GWB_UINTX) S = gwb::uintx_gemv_splits(K, (int)B);
  if (is_mxfp4(sp->format)) S = gwb::mxfp4_gemv_splits(K, (int)B);
  return S > 1 ? (size_t)S * (size_t)B * (size_t)N * sizeof(float) : 0;
}

// Enough for either path: the tile path is taken only when the buffers' alignment
// allows it, which the size query cannot know.
// The index-order GPTQ spec that group-ordered GPTQ is read as once its activations are
// gathered, and the workspace bytes of those gathered activations (bf16 [B, K]).
static gwb_qspec index_twin(const gwb_qspec* sp) {
  gwb_qspec t = *sp;
  t.format = sp->format == GWB_GPTQ_SYM_GROUPED ? GWB_GPTQ_SYM : GWB_GPTQ_ASYM;
  return t;
}
static size_t gathered_x_bytes(int64_t B, int64_t K) { return ((size_t)(B * K * 2) + 255) / 256 * 256; }

static size_t gemv_workspace(const gwb_qspec* sp, int64_t N, int64_t K, int64_t B) {
  if (is_grouped(sp->format)) {
    const gwb_qspec t = index_twin(sp);
    return gathered_x_bytes(B, K) + gemv_workspace(&t, N, K, B);
  }
  const size_t a = gemv_kernel_workspace(sp, N, K, B);
  if (gemv_uintx_via_decode(sp, N, K, B)) {
    const size_t b = gwb::uintx_decode_workspace_bytes(sp->nbits, B, N, K);
    return a > b ? a : b;
  }
  if (!gemv_shape_via_gemm(sp, N, K, B)) return a;
  const size_t b = gwb::gemm_workspace_bytes(!is_mxfp4(sp->format), sp->group, B, N, K);
  return a > b ? a : b;
}

static int check_gemv(const gwb_qspec* sp, int64_t N, int64_t K, int64_t B) {
  if (int rc = check_spec(sp, N, K)) return rc;
  if (sp->format == GWB_UINTX && !gwb::uintx_gemv_supported(N, K))
    return fail(GWB_E_UNSUPPORTED, "the uintx GEMV needs N %% 8 == 0 and K %% 512 == 0, got N=%lld K=%lld",
                (long long)N, (long long)K);
  if (B < 1 || B > 8) return fail(GWB_E_ARG, "B must be 1..8, got %lld", (long long)B);
  return GWB_OK;
}

int gwb_gemv_workspace(const gwb_qspec* spec, int64_t N, int64_t K, int64_t B, size_t* bytes) {
  if (!bytes) return fail(GWB_E_ARG, "bytes is NULL");
  if (int rc = check_gemv(spec, N, K, B)) return rc;
  *bytes = gemv_workspace(spec, N, K, B);
  return ok();
}

// gwb_gemv's kernels for validated arguments (x 16-byte aligned, workspace as needed).
static int gemv_dispatch(const gwb_qspec* spec, const gwb_qtensors* w, int64_t N, int64_t K, const void* x, int64_t B,
                         int64_t ldx, void* y, int32_t y_dtype, int64_t ldy, void* workspace, hipStream_t st) {
  const bool tiles = gemv_shape_via_gemm(spec, N, K, B) && aligned16(y) && ldy % 8 == 0 && B * ldx < kMaxElems &&
                     aligned16(w->codes) && aligned16(w->scales);
  if (gemv_uintx_via_decode(spec, N, K, B) && aligned16(w->codes) && aligned16(w->scales) && aligned16(w->zeros))
    gwb::launch_uintx_decode(spec->nbits, spec->group, w->codes, w->scales, w->zeros, N, K, x, B, ldx, y, y_dtype,
                             ldy, workspace, st);
  else if (tiles && is_mxfp4(spec->format))
    gwb::launch_mxfp4_gemm(w->codes, w->scales, N, K, x, B, ldx, y, y_dtype, ldy, workspace, st);
  else if (tiles)
    gwb::launch_gptq_gemm(spec->format == GWB_GPTQ_SYM, spec->group, w->codes, w->scales, w->zeros, N, K, x, B, ldx,
                          y, y_dtype, ldy, workspace, st);
  else if (is_mxfp4(spec->format))
    gwb::launch_mxfp4_gemv((int)B, w->codes, w->scales, N, K, x, ldx, y, y_dtype, ldy, (float*)workspace, st);
  else if (is_act(spec->format))
    gwb::launch_gptq_act_gemv(is_gptq_sym(spec->format), spec->group, (int)B, w->codes, w->scales, w->zeros,
                              (const int32_t*)w->g_idx, N, K, x, ldx, y, y_dtype, ldy, (float*)workspace, st);
  else if (spec->format == GWB_UINTX)
    gwb::launch_uintx_gemv(spec->nbits, spec->w_dtype, spec->group, (int)B, w->codes, w->scales, w->zeros, N, K, x,
                           ldx, y, y_dtype, ldy, (float*)workspace, st);
  else
    gwb::launch_gptq_gemv(spec->format == GWB_GPTQ_SYM, spec->group, (int)B, w->codes, w->scales, w->zeros, N, K, x,
                          ldx, y, y_dtype, ldy, (float*)workspace, st);
  return hip_check("gemv launch");
}

int gwb_gemv(const gwb_qspec* spec, const gwb_qtensors* w, int64_t N, int64_t K, const void* x, int64_t B,
             int64_t ldx, void* y, int32_t y_dtype, int64_t ldy, void* workspace, size_t workspace_bytes,
             void* stream) {
  if (int rc = check_gemv(spec, N, K, B)) return rc;
  if (y_dtype != GWB_F32 && y_dtype != GWB_BF16) return fail(GWB_E_ARG, "unknown y_dtype %d", y_dtype);
  if (N == 0) return ok();
  if (!x || !y) return fail(GWB_E_ARG, "x and y are required");
  if (ldx < K || ldy < N) return fail(GWB_E_ARG, "ldx must be >= K and ldy >= N");
  if (!aligned16(x) || ldx % 8) return fail(GWB_E_UNSUPPORTED, "x and its row stride must be 16-byte aligned");
  if (K == 0) return fail(GWB_E_SHAPE, "K must be positive");
  if (int rc = check_tensors(spec, w)) return rc;
  const size_t need = gemv_workspace(spec, N, K, B);
  if (need && (!workspace || workspace_bytes < need))
    return fail(GWB_E_SIZE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (need && !aligned16(workspace)) return fail(GWB_E_UNSUPPORTED, "workspace must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  if (is_grouped(spec->format)) {
    // group order: the activations gathered by the permutation, then index-order GPTQ
    gwb::launch_gather_columns(x, ldx, B, K, (const int32_t*)w->g_idx, workspace, st);
    const gwb_qspec t = index_twin(spec);
    return gemv_dispatch(&t, w, N, K, workspace, B, K, y, y_dtype, ldy,
                         (char*)workspace + gathered_x_bytes(B, K), st);
  }
  return gemv_dispatch(spec, w, N, K, x, B, ldx, y, y_dtype, ldy, workspace, st);
}

static int check_gemm(const gwb_qspec* sp, int64_t N, int64_t K, int64_t M) {
  if (int rc = check_spec(sp, N, K)) return rc;
  if (sp->format == GWB_UINTX && !gemm_uintx_shape(sp, N, K))
    return fail(GWB_E_UNSUPPORTED, "the uintx GEMM takes bf16 weights with N %% 8 == 0 and K %% 512 == 0");
  if (sp->format != GWB_GPTQ_SYM && sp->format != GWB_GPTQ_ASYM && !is_grouped(sp->format) && !is_mxfp4(sp->format) &&
      sp->format != GWB_UINTX)
    return fail(GWB_E_UNSUPPORTED,
                "the GEMM takes GPTQ (sym, asym, groups in index order or group order), MXFP4 and uintx weights");
  if (N % 8 || K % 128)
    return fail(GWB_E_UNSUPPORTED, "the GEMM needs N %% 8 == 0 and K %% 128 == 0, got N=%lld K=%lld", (long long)N,
                (long long)K);
  if (M < 0 || M > gwb::kGemmMaxRows) return fail(GWB_E_ARG, "M must be 0..%d, got %lld", gwb::kGemmMaxRows, (long long)M);
  if (M * K >= kMaxElems) return fail(GWB_E_UNSUPPORTED, "M*K = %lld exceeds 2^31 elements", (long long)(M * K));
  return GWB_OK;
}

static size_t gemm_workspace(const gwb_qspec* sp, int64_t M, int64_t N, int64_t K) {
  if (is_grouped(sp->format)) {
    const gwb_qspec t = index_twin(sp);
    return gathered_x_bytes(M, K) + gemm_workspace(&t, M, N, K);
  }
  if (sp->format == GWB_UINTX) return gwb::uintx_gemm_workspace_bytes(M, N, K);
  return gwb::gemm_workspace_bytes(!is_mxfp4(sp->format), sp->group, M, N, K);
}

int gwb_gemm_workspace(const gwb_qspec* spec, int64_t N, int64_t K, int64_t M, size_t* bytes) {
  if (!bytes) return fail(GWB_E_ARG, "bytes is NULL");
  if (int rc = check_gemm(spec, N, K, M)) return rc;
  *bytes = gemm_workspace(spec, M, N, K);
  return ok();
}

int gwb_gemm(const gwb_qspec* spec, const gwb_qtensors* w, int64_t N, int64_t K, const void* x, int64_t M,
             int64_t ldx, void* y, int32_t y_dtype, int64_t ldy, void* workspace, size_t workspace_bytes,
             void* stream) {
  if (int rc = check_gemm(spec, N, K, M)) return rc;
  if (y_dtype != GWB_F32 && y_dtype != GWB_BF16) return fail(GWB_E_ARG, "unknown y_dtype %d", y_dtype);
  if (N == 0 || M == 0) return ok();
  if (K == 0) return fail(GWB_E_SHAPE, "K must be positive");
  if (!x || !y) return fail(GWB_E_ARG, "x and y are required");
  if (ldx < K || ldy < N) return fail(GWB_E_ARG, "ldx must be >= K and ldy >= N");
  if (!aligned16(x) || ldx % 8) return fail(GWB_E_UNSUPPORTED, "x and its row stride must be 16-byte aligned");
  if (!aligned16(y) || ldy % 8) return fail(GWB_E_UNSUPPORTED, "y must be 16-byte aligned with ldy %% 8 == 0");
  if (M * ldx >= kMaxElems) return fail(GWB_E_UNSUPPORTED, "M*ldx = %lld exceeds 2^31 elements", (long long)(M * ldx));
  if (int rc = check_tensors(spec, w)) return rc;
  if (!aligned16(w->codes) || !aligned16(w->scales))
    return fail(GWB_E_UNSUPPORTED, "the GEMM needs 16-byte aligned codes and scales");
  const size_t need = gemm_workspace(spec, M, N, K);
  if (need && (!workspace || workspace_bytes < need))
    return fail(GWB_E_SIZE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (need && !aligned16(workspace)) return fail(GWB_E_UNSUPPORTED, "workspace must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  if (is_grouped(spec->format)) {
    // group order: the activation rows gathered by the permutation, then index-order GPTQ
    gwb::launch_gather_columns(x, ldx, M, K, (const int32_t*)w->g_idx, workspace, st);
    x = workspace;
    ldx = K;
    workspace = (char*)workspace + gathered_x_bytes(M, K);
  }
  if (spec->format == GWB_UINTX)
    gwb::launch_uintx_gemm(spec->nbits, spec->group, w->codes, w->scales, w->zeros, N, K, x, M, ldx, y, y_dtype, ldy,
                           workspace, st);
  else if (is_mxfp4(spec->format))
    gwb::launch_mxfp4_gemm(w->codes, w->scales, N, K, x, M, ldx, y, y_dtype, ldy, workspace, st);
  else
    gwb::launch_gptq_gemm(is_gptq_sym(spec->format), spec->group, w->codes, w->scales, w->zeros, N, K, x, M, ldx, y,
                          y_dtype, ldy, workspace, st);
  return hip_check("gemm launch");
}

// Host computation of the AWQ scaling table, the same steps and precision as the device
// table kernels: a' = max(a, 1e-8) in float32, then float64 for an = a' / mean(a'),
// p = clamp(an**alpha, 1e-2, 1e2) (exact 1, an and sqrt(an) for alpha 0, 1 and 0.5) and
// s = p / exp(mean(log p)), rounded once to float32.
int gwb_awq_scales_host(const float* a, int64_t K, const double* alphas, int32_t n_alpha, float* s_out) {
  if (!a || !alphas || !s_out) return fail(GWB_E_ARG, "a, alphas and s_out are required");
  if (K <= 0) return fail(GWB_E_ARG, "K must be positive, got %lld", (long long)K);
  if (n_alpha < 1 || n_alpha > 16) return fail(GWB_E_ARG, "n_alpha must be 1..16, got %d", n_alpha);
  std::vector<double> ap((size_t)K), p((size_t)K);
  double sum = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    ap[k] = (double)std::fmax(a[k], 1e-8f);
    sum += ap[k];
  }
  const double mean = sum / (double)K;
  for (int32_t i = 0; i < n_alpha; ++i) {
    const double alpha = alphas[i];
    double lg = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double an = ap[k] / mean;
      double v = alpha == 0.0 ? 1.0 : (alpha == 1.0 ? an : (alpha == 0.5 ? std::sqrt(an) : std::pow(an, alpha)));
      v = std::fmin(std::fmax(v, 1e-2), 1e2);
      p[k] = v;
      lg += std::log(v);
    }
    const double g = std::exp(lg / (double)K);
    for (int64_t k = 0; k < K; ++k) s_out[(int64_t)i * K + k] = (float)(p[k] / g);
  }
  return ok();
}

// ------------------------------------------------------------ allocation-free SNR
// gwb_quantize_snr_static keeps the per-block partial sums of the fused pass (and the
// code buffer of the two-call fallback, where it fits) in this file-scope device array
// instead of a caller workspace. Each device the library runs on holds its own copy
// until the process ends. The array's name is a host-side stand-in: host code never
// passes it to a kernel; it passes the device address hipGetSymbolAddress returns,
// looked up once per device on that device's first call (with the device current) and
// kept per device. Every call on one device shares that copy, so calls that overlap on
// one GPU race. Nothing in it needs to start at zero: each launch writes every partial
// (or code) that it later reads.
static __device__ __align__(256) unsigned char scratch[GWB_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int device_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(GWB_E_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(GWB_E_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(GWB_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return GWB_OK;
}
}  // namespace

int gwb_quantize_snr_static(const gwb_qspec* spec, const void* W, int64_t N, int64_t K, int64_t ldw,
                            const gwb_qtensors* out, double* d_out, void* stream) {
  if (int rc = check_spec(spec, N, K, true)) return rc;
  const gwb_sizes sz = sizes_of(spec, N, K);
  if (sz.workspace > (size_t)GWB_STATIC_SCRATCH_BYTES)
    return fail(GWB_E_SIZE, "this shape needs %zu bytes of scratch; the static array holds %d", sz.workspace,
                GWB_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (int rc = device_scratch(&ws)) return rc;
  return gwb_quantize_snr(spec, W, N, K, ldw, out, d_out, ws, (size_t)GWB_STATIC_SCRATCH_BYTES, stream);
}

int gwb_stream_bench(int32_t pattern, int32_t blocks, void* d_dst, const void* d_src, size_t bytes, void* stream) {
  if (!d_dst || !d_src) return fail(GWB_E_ARG, "NULL pointer");
  const int kind = pattern & 3;
  if (pattern < 0 || pattern > (GWB_STREAM_STRIDED | 3)) return fail(GWB_E_ARG, "unknown stream pattern %d", pattern);
  if (blocks < 1 || blocks > 65536) return fail(GWB_E_ARG, "blocks must be 1..65536, got %d", blocks);
  if (bytes % 64 || !aligned16(d_dst) || !aligned16(d_src))
    return fail(GWB_E_UNSUPPORTED, "stream needs 16-byte aligned pointers and a multiple of 64 bytes");
  if (kind == 1 && (size_t)blocks * 1024 > bytes)
    return fail(GWB_E_SIZE, "the read pattern writes blocks * 1024 bytes; %zu given", bytes);
  if (bytes == 0) return ok();
  gwb::launch_stream_bench(kind, (pattern & GWB_STREAM_STRIDED) != 0, (unsigned)blocks, d_dst, d_src, bytes / 16,
                           (hipStream_t)stream);
  return hip_check("stream launch");
}

}  // extern "C"
