"""Reconstruction SNR oracle (test infrastructure only).

Page export_gptq_cpu.py (quantize_sym / quantize_asym) reports
20 log10(||w|| / max(||w - deq||, 1e-12)); page quantize_dflash_mxfp4.py (main) reports
the relative error ||deq - w|| / ||w||, which is 10**(-SNR/20).
Here w is the float32 input, deq the float32 value of the dequantized stored tensors,
w - deq a float32 subtraction, and the sums of squares are float64.
"""
from __future__ import annotations

import math

import numpy as np


def sums(w, deq):
    """-> (sum w**2, sum (w - deq)**2) in float64."""
    w = np.asarray(w, np.float32)
    d = np.asarray(deq, np.float32)
    diff = (w - d).astype(np.float64)
    w64 = w.astype(np.float64)
    return float(np.sum(w64 * w64)), float(np.sum(diff * diff))


def snr_db_from_sums(sum_w2: float, sum_e2: float) -> float:
    """10 log10(sum_w2 / max(sum_e2, 1e-24)); equal to the page's form with norms,
    since max(||e||, 1e-12)**2 = max(||e||**2, 1e-24). -inf for an all-zero w."""
    if sum_w2 == 0.0:
        return -math.inf
    return 10.0 * math.log10(sum_w2 / max(sum_e2, 1e-24))


def snr_db(w, deq) -> float:
    return snr_db_from_sums(*sums(w, deq))


def rel_error(sum_w2: float, sum_e2: float) -> float:
    return math.sqrt(sum_e2) / math.sqrt(sum_w2)
