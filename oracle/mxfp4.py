"""OCP MXFP4 oracle (test infrastructure only).

Follows page quantize_dflash_mxfp4.py: the E2M1 table, quantize_mxfp4 and
dequantize_mxfp4. Two readings differ from the page's literal code:

  * ties: the page's docstring, its comment and its Quark config all say round half to
    even; its code picks the first tied index and then rounds that index down to even,
    which sends 0.75 to 0.0 and 3.5 to 2.0 (neither neighbour). This oracle rounds to
    the nearest magnitude with ties to the even code. ties="page_literal" reproduces
    the page's code for documentation only.
  * exponent: the page takes floor(log2(amax)) in float32, which returns one too many
    for a float32 amax one ulp below a power of two. This oracle uses the exact
    unbiased exponent of amax (what the page's comment asks for: the block maximum
    lands at the top of the e2m1 range). Identical for bfloat16 inputs.
"""
from __future__ import annotations

import numpy as np

from ._fp import f32

# e2m1 magnitudes by 3-bit index; bit 3 of a code is the sign.
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
GROUP = 32


def block_exponent(amax: np.ndarray) -> np.ndarray:
    """e = floor(log2(amax)) - 2, or 0 for an all-zero block, clamped to [-127, 127].
    floor(log2(a)) is the exact unbiased exponent of a (frexp gives a = f * 2**E with
    f in [0.5, 1), so floor(log2 a) = E - 1), subnormals included."""
    amax = f32(amax)
    _, E = np.frexp(amax)
    e = np.where(amax > 0, (E.astype(np.int64) - 1) - 2, 0)
    return np.clip(e, -127, 127)


def nearest_index(mag: np.ndarray, ties: str = "even") -> np.ndarray:
    """Index into E2M1 of the nearest magnitude to each mag (0 <= mag <= 6).
    Distances are exact in float64 (mag is a float32)."""
    d = np.abs(mag.astype(np.float64)[..., None] - E2M1)
    best = d.min(axis=-1, keepdims=True)
    tied = d == best
    first = np.argmax(tied, axis=-1)            # lowest index at minimal distance
    two = tied.sum(axis=-1) > 1                 # two neighbours equally near
    if ties == "even":
        # the tied pair is (first, first + 1): keep whichever index is even
        idx = np.where(two, first + (first % 2), first)
    elif ties == "page_literal":
        idx = np.where(two, (first // 2) * 2, first)
    else:
        raise ValueError(ties)
    return idx.astype(np.uint8)


def quantize(w, ties: str = "even", chunk_rows: int = 256):
    """[N, K] float -> (packed uint8 [N, K/2], e8m0 uint8 [N, K/32]).

    Per block of 32 along K: amax = max |x|; e = block_exponent(amax); v = x / 2**e
    (float32, exact); sign = signbit(v); mag = min(|v|, 6); index = nearest e2m1
    magnitude; code = index | sign << 3; two codes per byte, the even K position in the
    low nibble; e8m0 = e + 127. Rows are processed in chunks only to bound memory, as
    the page does (its rows are independent)."""
    x = f32(w)
    assert x.ndim == 2 and x.shape[1] % GROUP == 0, x.shape
    n, k = x.shape
    packed = np.empty((n, k // 2), np.uint8)
    e8m0 = np.empty((n, k // GROUP), np.uint8)
    for r0 in range(0, n, chunk_rows):
        xb = x[r0:r0 + chunk_rows].reshape(-1, k // GROUP, GROUP)
        amax = np.abs(xb).max(axis=-1)
        e = block_exponent(amax)
        scale = np.ldexp(np.float32(1.0), e.astype(np.int32)).astype(np.float32)  # 2**e exactly
        v = xb / scale[..., None]
        sign = np.signbit(v)
        mag = np.minimum(np.abs(v), np.float32(E2M1_MAX))
        code = nearest_index(mag, ties) | (sign.astype(np.uint8) << 3)
        code = code.reshape(-1, k)
        packed[r0:r0 + chunk_rows] = code[:, 0::2] | (code[:, 1::2] << 4)
        e8m0[r0:r0 + chunk_rows] = (e + 127).astype(np.uint8)
    return packed, e8m0


def unpack_codes(packed) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    n, h = packed.shape
    code = np.empty((n, 2 * h), np.uint8)
    code[:, 0::2] = packed & 0xF
    code[:, 1::2] = packed >> 4
    return code


def dequantize(packed, e8m0, k: int) -> np.ndarray:
    """-> float32 [N, K]: +-E2M1[code & 7] * 2**(e8m0 - 127) (sign from bit 3, so a
    code of 8 gives -0.0). 2**(e8m0 - 127) is formed exactly (2**128 -> inf, as the
    page's float32 exp2 gives)."""
    code = unpack_codes(packed)
    assert code.shape[1] == k
    n = code.shape[0]
    mag = E2M1.astype(np.float32)[code & 7]
    val = np.where((code & 8) > 0, -mag, mag)
    with np.errstate(over="ignore"):
        scale = np.ldexp(np.float32(1.0), np.asarray(e8m0, np.int32) - 127).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):   # 2^128 (byte 255) times E2M1: inf, 0 * inf: NaN
        out = val.reshape(n, k // GROUP, GROUP) * scale[..., None]
    return out.reshape(n, k).astype(np.float32)
