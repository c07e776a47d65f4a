"""Exact rational re-derivations used to pin the oracle (independent of oracle/).

Every float operation of the method is one IEEE rounding of an exact result; these
helpers compute the exact result with fractions.Fraction and round it to a binary
format with a small, separately written round-to-nearest-even.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

INF = float("inf")


def pow2(e: int) -> Fraction:
    return Fraction(2) ** e


def floor_log2(a: Fraction) -> int:
    """Exact floor(log2(a)) for a > 0."""
    assert a > 0
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while pow2(e) > a:
        e -= 1
    while pow2(e + 1) <= a:
        e += 1
    return e


def rint_even(q: Fraction) -> int:
    """Nearest integer, ties to even."""
    n = math.floor(q)
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def round_binary(x: Fraction, p: int, emin: int, emax: int):
    """Round x to the nearest binary float with p significant bits, normal exponents
    [emin, emax], gradual underflow; ties to even. Returns a Fraction, or +-INF on
    overflow."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = max(floor_log2(a), emin)
    ulp = pow2(e - p + 1)
    v = rint_even(a / ulp) * ulp
    if v >= pow2(emax + 1):
        return sign * INF
    return sign * v


def rn32(x: Fraction):
    return round_binary(x, 24, -126, 127)


def rnbf16(x: Fraction):
    return round_binary(x, 8, -126, 127)


def rnf16(x: Fraction):
    return round_binary(x, 11, -14, 15)


def F(v) -> Fraction:
    """Exact value of a finite float (Python float or numpy float32)."""
    return Fraction(float(v))


def is_neg(v) -> bool:
    return math.copysign(1.0, float(v)) < 0


def f32_bits(v) -> int:
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


# ---------------------------------------------------------------- MXFP4, exactly
E2M1_EXACT = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
              Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def mxfp4_block_exact(values):
    """32 floats -> (codes list, e). Nearest e2m1 magnitude of |x| / 2**e by exact
    distance; on an exact tie the even index; sign bit from the float's sign (so -0.0
    and negatives that round to zero keep it)."""
    amax = max(abs(F(v)) for v in values)
    e = floor_log2(amax) - 2 if amax > 0 else 0
    e = min(max(e, -127), 127)
    codes = []
    for v in values:
        m = min(abs(F(v)) / pow2(e), Fraction(6))
        d = [abs(m - g) for g in E2M1_EXACT]
        best = min(d)
        cand = [i for i, di in enumerate(d) if di == best]
        idx = cand[0] if len(cand) == 1 else [i for i in cand if i % 2 == 0][0]
        codes.append(idx | (8 if is_neg(v) else 0))
    return codes, e


def mxfp4_dequant_exact(code: int, e8m0: int) -> Fraction:
    m = E2M1_EXACT[code & 7] * pow2(e8m0 - 127)
    return -m if code & 8 else m


def same(v, want) -> bool:
    """v (a float) equals want (a Fraction, or +-INF) exactly."""
    v = float(v)
    if isinstance(want, float):
        return v == want
    return math.isfinite(v) and Fraction(v) == want
