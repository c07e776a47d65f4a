"""Pins for the AWQ fold + requantize oracle (page quantize_dflash_mxfp4.py, main and
its module docstring: norm / s, columns * s, up rows / s, each rounded to bfloat16,
then quantize_mxfp4 of the folded weight)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle.fold as fold
import oracle.mxfp4 as mx
from _exact import F, mxfp4_block_exact, rnbf16
from group_wise_bit_amd import workloads


def _bf16_weight(n, k, seed):
    return workloads.mxfp4_weight(n, k, seed=seed).float().numpy()


def _scales(k, seed, lo=-2.0, hi=2.0):
    return np.exp(np.random.default_rng(seed).uniform(lo, hi, k)).astype(np.float32)


def test_each_step_is_one_rounding_of_the_exact_result():
    """Brute force with exact rationals: column step, then row step, each the bf16
    rounding (RNE) of the exact product or quotient of the previous bf16 value."""
    w = _bf16_weight(6, 32, 81)
    c, r = _scales(32, 82), _scales(6, 83)
    for col_op in ("mul", "div"):
        for row_op in ("none", "mul", "div"):
            got = fold.fold(w, c, col_op, r if row_op != "none" else None, row_op)
            for i in range(6):
                for j in range(32):
                    v = F(w[i, j])
                    v = rnbf16(v * F(c[j]) if col_op == "mul" else v / F(c[j]))
                    if row_op == "mul":
                        v = rnbf16(v * F(r[i]))
                    elif row_op == "div":
                        v = rnbf16(v / F(r[i]))
                    assert Fraction(float(got[i, j])) == v, (col_op, row_op, i, j)


def test_unit_scales_are_the_identity():
    w = _bf16_weight(16, 64, 84)
    ones_c, ones_r = np.ones(64, np.float32), np.ones(16, np.float32)
    for op in ("mul", "div"):
        assert np.array_equal(fold.fold(w, ones_c, op, ones_r, op), w)
    x, packed, e8 = fold.fold_quantize(w, ones_c, "mul")
    p0, e0 = mx.quantize(w)
    assert np.array_equal(packed, p0) and np.array_equal(e8, e0)


def test_powers_of_two_scale_exactly_and_shift_the_block_exponent():
    """s = 2^m per column scales every value exactly (in range), so a uniform s = 2^m
    keeps every MXFP4 code and adds m to every E8M0 byte."""
    w = _bf16_weight(24, 96, 85)
    m = np.random.default_rng(86).integers(-5, 6, 96)
    c = (2.0 ** m).astype(np.float32)
    assert np.array_equal(fold.fold(w, c, "mul"), w * c[None, :])
    assert np.array_equal(fold.fold(w, c, "div"), w / c[None, :])
    for shift in (-3, 4):
        x, packed, e8 = fold.fold_quantize(w, np.full(96, 2.0 ** shift, np.float32), "mul")
        p0, e0 = mx.quantize(w)
        assert np.array_equal(packed, p0)
        assert np.array_equal(e8.astype(int), e0.astype(int) + shift)


def test_multiply_then_divide_by_a_power_of_two_is_the_identity():
    w = _bf16_weight(8, 64, 87)
    r = (2.0 ** np.random.default_rng(88).integers(-4, 5, 8)).astype(np.float32)
    c = (2.0 ** np.random.default_rng(89).integers(-4, 5, 64)).astype(np.float32)
    x = fold.fold(fold.fold(w, c, "mul", r, "mul"), c, "div", r, "div")
    assert np.array_equal(x, w)


def test_orientation_and_order():
    """Column values broadcast along rows and row values along columns; the column
    step comes first (two roundings: (x * c) then / r, not x * (c / r))."""
    w = np.zeros((2, 32), np.float32)
    w[0, 1], w[1, 4] = 1.0, 3.0
    c = np.ones(32, np.float32)
    c[1], c[4] = 3.0, 5.0
    r = np.array([7.0, 11.0], np.float32)
    x = fold.fold(w, c, "mul", r, "div")
    assert Fraction(float(x[0, 1])) == rnbf16(rnbf16(Fraction(3)) / 7)
    assert Fraction(float(x[1, 4])) == rnbf16(rnbf16(Fraction(15)) / 11)
    assert np.count_nonzero(x) == 2


def test_requantize_is_mxfp4_of_the_folded_bf16_values():
    w = _bf16_weight(4, 64, 90)
    c = _scales(64, 91)
    x, packed, e8 = fold.fold_quantize(w, c, "mul")
    for i in range(4):
        for b in range(2):
            codes, e = mxfp4_block_exact([x[i, 32 * b + t] for t in range(32)])
            assert e8[i, b] == e + 127
            got = [(packed[i, 16 * b + t // 2] >> (4 * (t % 2))) & 0xF for t in range(32)]
            assert got == codes


def test_rejects_mismatched_vectors():
    w = _bf16_weight(4, 32, 92)
    with pytest.raises(AssertionError):
        fold.fold(w, np.ones(31, np.float32), "mul")
    with pytest.raises(AssertionError):
        fold.fold(w, None, "none", np.ones(3, np.float32), "div")
