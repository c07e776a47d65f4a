"""AWQ-style alpha search on MXFP4 (test infrastructure only).

Follows page quantize_dflash_mxfp4.py, search_scale, with the objective its module
docstring defines: the diagonal surrogate ||(Wq / s - W) diag(a)||_F, a = per-input-
channel mean |x|, s a per-column scaling searched over alpha.

Steps:
  rows: when N > max_rows, W_sub = W[::max(1, N // max_rows)][:max_rows]
  a' = max(a, 1e-8) (float32);  an = a' / mean(a')
  for alpha in the grid (default 0, 0.1, ..., 1.0):
      s = clamp(an ** alpha, 1e-2, 1e2);  s = s / exp(mean(log s))   (geometric mean 1)
      X = W_sub * s;  D = dequantize(quantize_mxfp4(X))
      err = sum(((D / s - W_sub) * a') ** 2)
  best = the first alpha with the strictly smallest err

Readings: the s table is computed in float64 and rounded once to float32 (the page
does it with float32 torch ops whose pow/log/exp/mean rounding is unspecified);
D / s, the subtraction, the product with a' and the square are float32 ops as on the
page; the sum is accumulated in float64 (the page's float32 sum has no fixed order).
"""
from __future__ import annotations

import numpy as np

from . import mxfp4
from ._fp import f32

DEFAULT_ALPHAS = tuple(i / 10 for i in range(11))


def subsample_rows(w, max_rows: int = 2048):
    w = np.asarray(w)
    if w.shape[0] > max_rows:
        w = w[:: max(1, w.shape[0] // max_rows)][:max_rows]
    return w


def clamp_stat(a) -> np.ndarray:
    return np.maximum(f32(a), np.float32(1e-8))


def scale_table(a, alphas=DEFAULT_ALPHAS) -> np.ndarray:
    """-> float32 [len(alphas), K]."""
    a64 = clamp_stat(a).astype(np.float64)
    an = a64 / np.mean(a64)
    rows = []
    for alpha in alphas:
        s = np.clip(an ** float(alpha), 1e-2, 1e2)
        s = s / np.exp(np.mean(np.log(s)))
        rows.append(s.astype(np.float32))
    return np.stack(rows)


def weighted_error(w_sub, a, s) -> float:
    """sum(((D / s - W) * a') ** 2) for one float32 scaling row s."""
    W = f32(w_sub)
    a32 = clamp_stat(a)
    s = f32(s)
    X = W * s
    packed, e8m0 = mxfp4.quantize(X)
    D = mxfp4.dequantize(packed, e8m0, W.shape[1])
    t = (D / s - W) * a32
    t2 = t * t                                   # float32 square
    return float(np.sum(t2.astype(np.float64)))


def search(w, a, alphas=DEFAULT_ALPHAS, max_rows: int = 2048):
    """-> dict(errors float64 [n_alpha], best index, best_alpha, s_table)."""
    W = f32(subsample_rows(w, max_rows))
    table = scale_table(a, alphas)
    errs = np.array([weighted_error(W, a, table[i]) for i in range(len(alphas))])
    best = None
    for i, e in enumerate(errs):
        if best is None or e < errs[best]:
            best = i
    return dict(errors=errs, best=best, best_alpha=alphas[best], s_table=table)
