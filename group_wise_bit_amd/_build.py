"""Build libgwb.so in-tree with hipcc for gfx950.

    python -m group_wise_bit_amd._build

Objects go to group_wise_bit_amd/_build/, the library to group_wise_bit_amd/libgwb.so.
Device code is compiled without floating-point contraction (every float op is one
IEEE rounding, as the pages' step lists require), with IEEE division and denormals
kept, and with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgwb.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.hip", "common.hip", "mxfp4.hip", "gptq.hip", "gptq_act.hip", "uintx.hip", "uintx_bf16.hip", "uintx_f16.hip", "uintx_f32.hip",
           "uintx_flat.hip", "awq.hip", "fold.hip", "gemv.hip", "gemm.hip"]
# The tiled uintx kernels are compiled without NaN semantics, which lets the compiler
# fold each float min/max into its DPP exchange instead of quieting every operand first
# (measured: the fused uintx quantize+SNR passes run about 7% faster). No NaN reaches a
# min, max, median or select in these files when the weights are finite (non-finite
# weights are outside the method and untested):
#   * the group extremes run on keys built from the weight words, and a finite weight's
#     word never reads as a NaN (its exponent field is not all ones);
#   * the scale is a rounded difference of finite extremes over qmax, at least 2^-23; it
#     may round to +inf for float16 weights, and inf / qmax, max(inf, 2^-23), x / inf and
#     1 / inf are not NaN;
#   * the code is med3(rint(w * inv), -zp, qmax - zp) with inv finite (an infinite float16
#     reciprocal is decided on its bits before any arithmetic, see ux_inv_is_inf), so the
#     product is finite or +-inf;
#   * dequantized values r((q - zp) * s) can be NaN (0 * inf, an overflowed float16
#     scale), like the page's; they only feed stores and the error sums' additions, whose
#     float64/float32 fallback choice depends on the extremes alone.
EXTRA = {name: ["-fno-honor-nans"] for name in ("uintx.hip", "uintx_bf16.hip", "uintx_f16.hip", "uintx_f32.hip")}
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # hipcc's host pass does not know the packed-fp32 feature; that warning is expected
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    return r.returncode, "\n".join(lines)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        rc, out = _run([HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        return src, obj, rc, out

    jobs = min(len(SOURCES), max(1, os.cpu_count() or 1), 8)
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(compile_one, SOURCES))
    failed = [r for r in results if r[2] != 0]
    for src, _, rc, out in results:
        if out and (verbose or rc):
            print(f"[{src}]\n{out}", file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed for " + ", ".join(r[0] for r in failed))
    tmp = LIB + ".tmp"
    # --no-undefined: a kernel whose host-side launch stub went missing fails here, not at load
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp,
                    *[r[1] for r in results]])
    if rc:
        raise RuntimeError("link failed:\n" + out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
