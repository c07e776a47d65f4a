"""Folding AWQ scales into weights, then requantizing (test infrastructure only).

Follows page quantize_dflash_mxfp4.py, main and its module docstring. After the alpha
search picks s, the page folds s into the tensors around each linear and then
quantizes every served linear to MXFP4:

  norm vector  [K]:     (norm.float() / s).to(bfloat16)          column divide
  linear       [N, K]:  (W.float() * s).to(bfloat16)             column multiply
                        (q, k, v, gate, up, down and the conv's kernel projection)
  up rows      [I, H]:  (up.float() / s_down[:, None]).to(bf16)  row divide, applied
                        after up's own column fold (so two bf16 roundings)
  then quantize_mxfp4 of the folded bf16 weight.

Each fold step is one float32 operation on the float32 widening of a bfloat16 value,
rounded to bfloat16 (RNE). Here a fold is an optional column step (multiply or divide
by col[k]) followed by an optional row step (multiply or divide by row[n]), each
rounded to bfloat16; the pages' cases are the column multiply, the column divide of a
one-row matrix (a norm vector) and the column multiply followed by a row divide (up).
"""
from __future__ import annotations

import numpy as np

from . import mxfp4
from ._fp import bf16_round, f32

OPS = ("none", "mul", "div")


def _apply(x, v, op: str):
    if op == "none" or v is None:
        return x
    if op == "mul":
        return bf16_round(x * v)
    if op == "div":
        return bf16_round(x / v)
    raise ValueError(op)


def fold(w, col=None, col_op: str = "none", row=None, row_op: str = "none") -> np.ndarray:
    """[N, K] weights (bf16 values, float32 carrier) -> folded [N, K] bf16 values."""
    x = f32(w)
    assert x.ndim == 2
    if col_op != "none":
        c = f32(col).reshape(1, -1)
        assert c.shape[1] == x.shape[1]
        x = _apply(x, c, col_op)
    if row_op != "none":
        r = f32(row).reshape(-1, 1)
        assert r.shape[0] == x.shape[0]
        x = _apply(x, r, row_op)
    return x


def fold_quantize(w, col=None, col_op: str = "none", row=None, row_op: str = "none"):
    """-> (folded bf16 values [N, K], packed [N, K/2], e8m0 [N, K/32])."""
    x = fold(w, col, col_op, row, row_op)
    packed, e8m0 = mxfp4.quantize(x)
    return x, packed, e8m0
