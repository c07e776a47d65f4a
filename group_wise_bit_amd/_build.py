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
# The uintx, GPTQ and AWQ arithmetic feeds no NaN to a float op whose result is kept
# (the one NaN uintx can make, a float16 zero weight times an infinite reciprocal, is
# decided on the reciprocal's bits first), and non-finite inputs are outside the method;
# without NaN semantics the compiler drops the canonicalization it otherwise inserts
# around every float min/max. (A NaN fp16 scale handed to GPTQ dequantization still
# yields NaN on either branch.)
EXTRA = {name: ["-fno-honor-nans"] for name in ("uintx.hip", "uintx_bf16.hip", "uintx_f16.hip", "uintx_f32.hip",
                                                "gptq.hip", "awq.hip")}
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
