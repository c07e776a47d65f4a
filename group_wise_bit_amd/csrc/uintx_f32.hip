// Tiled uintx kernels for float32 weights, groups 32, 64 and 128: instantiations of
// uintx_tiled.hpp (page uintx_quant.py, the arithmetic in the weight's dtype), compiled on
// their own so the library builds in parallel.
#include "uintx_tiled.hpp"

namespace gwb {

void uintx_tiled_quant_f32(int nbits, int group, const void* W, int64_t N, int64_t K, int64_t ldw, void* packed,
                           void* scales, void* zeros, double* part, hipStream_t st) {
  if (group == 32) ux_tiled_quant_entry<kF32, 32>(nbits, W, N, K, ldw, packed, scales, zeros, part, st);
  else if (group == 64) ux_tiled_quant_entry<kF32, 64>(nbits, W, N, K, ldw, packed, scales, zeros, part, st);
  else ux_tiled_quant_entry<kF32, 128>(nbits, W, N, K, ldw, packed, scales, zeros, part, st);
}

void uintx_tiled_dequant_f32(int nbits, int group, const void* packed, const void* scales, const void* zeros,
                             int64_t N, int64_t K, void* out, int32_t out_dtype, int64_t ldo, hipStream_t st) {
  if (group == 32) ux_tiled_dequant_entry<kF32, 32>(nbits, packed, scales, zeros, N, K, out, out_dtype, ldo, st);
  else if (group == 64) ux_tiled_dequant_entry<kF32, 64>(nbits, packed, scales, zeros, N, K, out, out_dtype, ldo, st);
  else ux_tiled_dequant_entry<kF32, 128>(nbits, packed, scales, zeros, N, K, out, out_dtype, ldo, st);
}

void uintx_tiled_err_f32(int nbits, int group, const void* W, int64_t N, int64_t K, int64_t ldw, const void* packed,
                         const void* scales, const void* zeros, double* part, hipStream_t st) {
  if (group == 32) ux_tiled_err_entry<kF32, 32>(nbits, W, N, K, ldw, packed, scales, zeros, part, st);
  else if (group == 64) ux_tiled_err_entry<kF32, 64>(nbits, W, N, K, ldw, packed, scales, zeros, part, st);
  else ux_tiled_err_entry<kF32, 128>(nbits, W, N, K, ldw, packed, scales, zeros, part, st);
}

void uintx_tiled_gemv_f32(int nbits, int group, int B, const void* packed, const void* scales, const void* zeros,
                          int64_t N, int64_t K, const void* x, int64_t ldx, GemvOut out, hipStream_t st) {
  if (group == 32) ux_tiled_gemv_entry<kF32, 32>(nbits, B, packed, scales, zeros, N, K, x, ldx, out, st);
  else if (group == 64) ux_tiled_gemv_entry<kF32, 64>(nbits, B, packed, scales, zeros, N, K, x, ldx, out, st);
  else ux_tiled_gemv_entry<kF32, 128>(nbits, B, packed, scales, zeros, N, K, x, ldx, out, st);
}

}  // namespace gwb
