"""Float helpers of the oracle (test infrastructure only).

bfloat16 values are carried as float32 arrays whose low 16 bits are zero.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32)


def bf16_round(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16, ties to even (bfloat16 keeps the
    top 16 bits of a float32). NaN stays NaN; overflow goes to +-inf."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    out = r.view(np.float32).reshape(x.shape)
    nan = np.isnan(x)
    if nan.any():
        out = np.where(nan, np.float32(np.nan), out)
    return out


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of float32 values that are exactly bfloat16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    assert not np.any(b & 0xFFFF), "value is not a bfloat16"
    return (b >> 16).astype(np.uint16)


def from_bf16_bits(u) -> np.ndarray:
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32)


def is_bf16(x) -> bool:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return not np.any(x.view(np.uint32) & 0xFFFF)
