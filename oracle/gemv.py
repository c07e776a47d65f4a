"""Dequantize-and-multiply reference for the decode GEMV and the prefill GEMM (test
infrastructure only; both consumers compute the same product, for B <= 8 or M rows).

Page export_gptq_cpu.py gives the reason for the 4-bit formats: in a decode step the
weight read dominates (its lm_head note: the 131072 x 2048 head is the single largest
read), and vLLM's W4A16 kernel consumes the GPTQ tensors directly. Page uintx_quant.py
(forward) and page quantize_dflash_mxfp4.py (served linears) consume their formats the
same way: y = x @ dequantize(W)^T.

The reference is that definition written out: the stored tensors dequantized by the
format oracles (every dequantized value is exact in float32), widened to float64 with
the bf16 activations, and multiplied in float64. For the sizes tested (K <= 2^14) the
float64 result is the exact product to within 2^-40 relative, far below the float32
accumulation error the device result is allowed (the bound is the tests' business).
"""
from __future__ import annotations

import numpy as np

from . import gptq, mxfp4, uintx
from ._fp import bf16_round, f32


def dequantized(fmt: str, q: dict, N: int, K: int, group=None, nbits: int = 4,
                dtype: str = "bf16") -> np.ndarray:
    """Stored tensors of one format -> the float32 [N, K] weight the consumer multiplies
    (group: the format's default, GPTQ 128 and uintx 64, when None).
    uintx (page uintx_quant.py, forward): the dequantized weight of the weight dtype,
    converted to the activations' bf16 when it is not bf16 already (`w.to(x.dtype)`)."""
    if fmt == "gptq_sym" or fmt == "gptq_asym":
        return gptq.dequantize(q["qweight"], q["scales"], q["qzeros"], 128 if group is None else group,
                               fmt == "gptq_sym")
    if fmt == "mxfp4":
        return mxfp4.dequantize(q["packed"], q["e8m0"], K)
    if fmt == "uintx":
        w = uintx.dequantize(q["packed"], q["scale_bytes"], q["zero_point"], nbits, N, K,
                             64 if group is None else group, dtype)
        return w if dtype == "bf16" else bf16_round(w)
    raise ValueError(fmt)


def gemv(deq, x) -> np.ndarray:
    """deq float32 [N, K], x [B, K] (bf16 values) -> float64 [B, N] = x @ deq^T."""
    d = np.asarray(deq, np.float64)
    xx = f32(x).astype(np.float64)
    if xx.ndim == 1:
        xx = xx[None, :]
    return xx @ d.T


def abs_gemv(deq, x) -> np.ndarray:
    """sum_k |deq[n, k] * x[b, k]| (float64), the scale of any accumulation error."""
    return np.abs(f32(x).astype(np.float64).reshape(-1, np.shape(deq)[1])) @ np.abs(np.asarray(deq, np.float64)).T
