// Affine uint2..uint7 (torchao-style, preserve_zero): the bfloat16 / group-64 tiled
// kernels (page uintx_quant.py's defaults) including the decode GEMV on packed uintx
// weights, and the launch selection for every dtype and group. Page uintx_quant.py: pack_uintx,
// unpack_uintx, UIntXQuantizer._quantize_impl, _dequantize_native and forward.
// The tiled kernels (uintx_tiled.hpp) need numel % 8G == 0; their other instantiations
// live in uintx_f16.hip, uintx_f32.hip and uintx_bf16.hip, and every other shape takes
// the two-pass path of uintx_flat.hip.
#include "device_common.hpp"
#include "kernels.hpp"
#include "uintx_layout.hpp"
#include "uintx_tiled.hpp"

namespace gwb {

// ------------------------------------------------------------------ launchers
bool uintx_tiled(int32_t dt, int group, int64_t N, int64_t K) {
  (void)dt;
  return uintx_tiles_fit(group, N * K);
}
size_t uintx_code_workspace(int32_t dt, int group, int64_t N, int64_t K) {
  return uintx_tiled(dt, group, N, K) ? 0 : (size_t)(N * K);
}

void launch_uintx_quant(int nbits, int32_t dt, int group, const void* W, int64_t N, int64_t K, int64_t ldw,
                        void* packed, void* scales, void* zeros, void* workspace, double* part, hipStream_t st) {
  if (!uintx_tiled(dt, group, N, K))
    launch_uintx_quant_flat(nbits, dt, group, W, N, K, ldw, packed, scales, zeros, workspace, st);
  else if (dt == kBF16 && group == 64)
    ux_tiled_quant_entry<kBF16, 64>(nbits, W, N, K, ldw, packed, scales, zeros, part, st);
  else if (dt == kBF16)
    uintx_tiled_quant_bf16(nbits, group, W, N, K, ldw, packed, scales, zeros, part, st);
  else if (dt == kF16)
    uintx_tiled_quant_f16(nbits, group, W, N, K, ldw, packed, scales, zeros, part, st);
  else
    uintx_tiled_quant_f32(nbits, group, W, N, K, ldw, packed, scales, zeros, part, st);
}

void launch_uintx_dequant(int nbits, int32_t dt, int group, const void* packed, const void* scales,
                          const void* zeros, int64_t N, int64_t K, void* out, int32_t out_dtype, int64_t ldo,
                          hipStream_t st) {
  if (!uintx_tiled(dt, group, N, K))
    launch_uintx_dequant_flat(nbits, dt, group, packed, scales, zeros, N, K, out, out_dtype, ldo, st);
  else if (dt == kBF16 && group == 64)
    ux_tiled_dequant_entry<kBF16, 64>(nbits, packed, scales, zeros, N, K, out, out_dtype, ldo, st);
  else if (dt == kBF16)
    uintx_tiled_dequant_bf16(nbits, group, packed, scales, zeros, N, K, out, out_dtype, ldo, st);
  else if (dt == kF16)
    uintx_tiled_dequant_f16(nbits, group, packed, scales, zeros, N, K, out, out_dtype, ldo, st);
  else
    uintx_tiled_dequant_f32(nbits, group, packed, scales, zeros, N, K, out, out_dtype, ldo, st);
}

// The tiled error kernels run one block per tile (their partials follow the tiles); the
// flat one is grid-stride with a capped grid. Both depend on the shape only.
unsigned uintx_err_blocks(int32_t dt, int group, int64_t N, int64_t K) {
  return uintx_tiled(dt, group, N, K) ? uintx_tiles(N * K) : uintx_flat_err_blocks(N, K);
}

void launch_uintx_err(int nbits, int32_t dt, int group, const void* W, int64_t N, int64_t K, int64_t ldw,
                      const void* packed, const void* scales, const void* zeros, double* part, hipStream_t st) {
  if (!uintx_tiled(dt, group, N, K))
    launch_uintx_err_flat(nbits, dt, group, W, N, K, ldw, packed, scales, zeros, part, st);
  else if (dt == kBF16 && group == 64)
    ux_tiled_err_entry<kBF16, 64>(nbits, W, N, K, ldw, packed, scales, zeros, part, st);
  else if (dt == kBF16)
    uintx_tiled_err_bf16(nbits, group, W, N, K, ldw, packed, scales, zeros, part, st);
  else if (dt == kF16)
    uintx_tiled_err_f16(nbits, group, W, N, K, ldw, packed, scales, zeros, part, st);
  else
    uintx_tiled_err_f32(nbits, group, W, N, K, ldw, packed, scales, zeros, part, st);
}

// ------------------------------------------------------------------ decode GEMV
int uintx_gemv_splits(int64_t K, int B) { return (int)(K / (512 * ux_gemv_chunks(K, B))); }

bool uintx_gemv_supported(int64_t N, int64_t K) { return N % 8 == 0 && K % 512 == 0; }

void launch_uintx_gemv(int nbits, int32_t dt, int group, int B, const void* packed, const void* scales,
                       const void* zeros, int64_t N, int64_t K, const void* x, int64_t ldx, void* y, int32_t y_dtype,
                       int64_t ldy, float* part, hipStream_t st) {
  // one split: each row's sum is complete in one wavefront and goes straight to y
  const int S = uintx_gemv_splits(K, B);
  const GemvOut out{part, y, ldy, S > 1 ? GemvOut::kPart : (y_dtype == kBF16 ? GemvOut::kBF16 : GemvOut::kF32)};
  if (dt == kBF16 && group == 64) ux_tiled_gemv_entry<kBF16, 64>(nbits, B, packed, scales, zeros, N, K, x, ldx, out, st);
  else if (dt == kBF16) uintx_tiled_gemv_bf16(nbits, group, B, packed, scales, zeros, N, K, x, ldx, out, st);
  else if (dt == kF16) uintx_tiled_gemv_f16(nbits, group, B, packed, scales, zeros, N, K, x, ldx, out, st);
  else uintx_tiled_gemv_f32(nbits, group, B, packed, scales, zeros, N, K, x, ldx, out, st);
  if (S > 1) launch_gemv_finalize(part, S, B, N, y, y_dtype, ldy, st);
}

}  // namespace gwb
