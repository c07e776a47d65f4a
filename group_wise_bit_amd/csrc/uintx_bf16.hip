// Tiled uintx kernels for bfloat16 weights, groups 32 and 128 (group 64 is in uintx.hip):
// instantiations of uintx_tiled.hpp (page uintx_quant.py, the arithmetic in the weight's
// dtype), compiled on their own so the library builds in parallel.
#include "uintx_tiled.hpp"

namespace gwb {

void uintx_tiled_quant_bf16(int nbits, int group, const void* W, int64_t N, int64_t K, int64_t ldw, void* packed,
                            void* scales, void* zeros, double* part, hipStream_t st) {
  if (group == 32) ux_tiled_quant_entry<kBF16, 32>(nbits, W, N, K, ldw, packed, scales, zeros, part, st);
  else ux_tiled_quant_entry<kBF16, 128>(nbits, W, N, K, ldw, packed, scales, zeros, part, st);
}

void uintx_tiled_dequant_bf16(int nbits, int group, const void* packed, const void* scales, const void* zeros,
                              int64_t N, int64_t K, void* out, int32_t out_dtype, int64_t ldo, hipStream_t st) {
  if (group == 32) ux_tiled_dequant_entry<kBF16, 32>(nbits, packed, scales, zeros, N, K, out, out_dtype, ldo, st);
  else ux_tiled_dequant_entry<kBF16, 128>(nbits, packed, scales, zeros, N, K, out, out_dtype, ldo, st);
}

void uintx_tiled_err_bf16(int nbits, int group, const void* W, int64_t N, int64_t K, int64_t ldw, const void* packed,
                          const void* scales, const void* zeros, double* part, hipStream_t st) {
  if (group == 32) ux_tiled_err_entry<kBF16, 32>(nbits, W, N, K, ldw, packed, scales, zeros, part, st);
  else ux_tiled_err_entry<kBF16, 128>(nbits, W, N, K, ldw, packed, scales, zeros, part, st);
}

void uintx_tiled_gemv_bf16(int nbits, int group, int B, const void* packed, const void* scales, const void* zeros,
                           int64_t N, int64_t K, const void* x, int64_t ldx, GemvOut out, hipStream_t st) {
  if (group == 32) ux_tiled_gemv_entry<kBF16, 32>(nbits, B, packed, scales, zeros, N, K, x, ldx, out, st);
  else ux_tiled_gemv_entry<kBF16, 128>(nbits, B, packed, scales, zeros, N, K, x, ldx, out, st);
}

}  // namespace gwb
