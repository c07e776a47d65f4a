"""Pins for the MXFP4 oracle (page quantize_dflash_mxfp4.py: E2M1 table, quantize_mxfp4,
dequantize_mxfp4). Everything here is checked against something other than the oracle:
a hand-derived worked example, exact rational brute force, invariants and closed forms."""
import numpy as np
import pytest
import torch

import oracle.mxfp4 as mx
from _exact import INF, F, floor_log2, rn32, mxfp4_block_exact, mxfp4_dequant_exact, pow2
from golden.golden import floats, hexbytes, load
from group_wise_bit_amd import workloads


def test_worked_example_block():
    g = load("mxfp4_worked_block.txt")
    x = np.array(floats(g["input_f32"]), np.float32)[None, :]
    packed, e8m0 = mx.quantize(x)
    assert packed.tobytes() == hexbytes(g["packed_hex"])
    assert e8m0.tolist() == [[int(g["e8m0"])]]
    lit, _ = mx.quantize(x, ties="page_literal")
    assert lit.tobytes() == hexbytes(g["packed_hex_page_literal"])


def test_ties_go_to_even_code():
    # the seven midpoints of the e2m1 magnitudes, in a block whose exponent is 0
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    x = np.zeros((1, 32), np.float32)
    x[0, :7] = mids
    x[0, 7] = 4.0          # amax 4 -> exp = 2 - 2 = 0
    code = mx.unpack_codes(mx.quantize(x)[0])[0, :7]
    assert code.tolist() == [0, 2, 2, 4, 4, 6, 6]
    lit = mx.unpack_codes(mx.quantize(x, ties="page_literal")[0])[0, :7]
    assert lit.tolist() == [0, 0, 2, 2, 4, 4, 6]


def _blocks_bruteforce(x):
    n, k = x.shape
    codes = np.empty((n, k), np.uint8)
    es = np.empty((n, k // 32), np.int64)
    for r in range(n):
        for b in range(k // 32):
            c, e = mxfp4_block_exact(x[r, 32 * b:32 * b + 32].tolist())
            codes[r, 32 * b:32 * b + 32] = c
            es[r, b] = e
    return codes, es


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_bruteforce_exact_random_and_adversarial(dtype):
    xs = [workloads.mxfp4_weight(4, 256, seed=11, dtype=dtype),
          workloads.adversarial_weight(8, 256, seed=12, dtype=dtype)]
    for t in xs:
        x = t.float().numpy()
        packed, e8m0 = mx.quantize(x)
        codes, es = _blocks_bruteforce(x)
        assert np.array_equal(mx.unpack_codes(packed), codes)
        assert np.array_equal(e8m0.astype(np.int64), es + 127)


def test_exponent_is_exact_below_power_of_two():
    # float32 amax one ulp below 8: exact floor(log2) is 2, so exp = 0 (e8m0 127);
    # a float32 log2 rounds to 3.0 here.
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = np.nextafter(np.float32(8.0), np.float32(0.0))
    _, e8m0 = mx.quantize(x)
    assert int(e8m0[0, 0]) == 127
    assert floor_log2(F(x[0, 0])) == 2


def test_invariants_block_max_lands_at_top():
    x = workloads.mxfp4_weight(16, 512, seed=13, dtype=torch.float32).numpy()
    packed, e8m0 = mx.quantize(x)
    code = mx.unpack_codes(packed).reshape(16, 16, 32)
    xb = x.reshape(16, 16, 32)
    amax_pos = np.abs(xb).argmax(-1)
    top = np.take_along_axis(code & 7, amax_pos[..., None], -1)[..., 0]
    assert set(np.unique(top)) <= {6, 7}
    amax = np.abs(xb).max(-1)
    for a, e in zip(amax.ravel(), e8m0.ravel()):
        assert int(e) == floor_log2(F(a)) + 125


def test_lossless_on_grid_blocks():
    rng = np.random.default_rng(14)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    x = np.empty((8, 128), np.float32)
    for r in range(8):
        for b in range(4):
            k = int(rng.integers(-30, 30))
            v = grid[rng.integers(0, 8, 32)] * rng.choice([-1, 1], 32)
            v[0] = rng.choice([4.0, 6.0])          # block max at the top binade
            x[r, 32 * b:32 * b + 32] = np.ldexp(v.astype(np.float32), k)
    packed, e8m0 = mx.quantize(x)
    d = mx.dequantize(packed, e8m0, 128)
    assert np.array_equal(d, x)


def test_zero_block_and_signed_zero():
    x = np.zeros((1, 64), np.float32)
    x[0, 32:] = -0.0
    packed, e8m0 = mx.quantize(x)
    assert e8m0.tolist() == [[127, 127]]
    assert packed[0, :16].tolist() == [0] * 16
    assert packed[0, 16:].tolist() == [0x88] * 16
    d = mx.dequantize(packed, e8m0, 64)
    assert np.all(d == 0) and np.all(np.signbit(d[0, 32:])) and not np.any(np.signbit(d[0, :32]))


def test_dequant_exact_all_codes_all_exponents():
    codes = np.arange(16, dtype=np.uint8)
    for e in list(range(0, 255)) + [255]:
        packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
        packed = np.tile(packed, 2)[None, :]                 # 32 codes
        d = mx.dequantize(packed, np.array([[e]], np.uint8), 32)[0]
        for i in range(32):
            c = int(codes[i % 16])
            if e == 255:
                if c & 7 == 0:
                    assert np.isnan(d[i])
                else:
                    assert np.isinf(d[i]) and (d[i] < 0) == bool(c & 8)
                continue
            want = rn32(mxfp4_dequant_exact(c, e))     # 6 * 2**127 overflows float32
            if abs(want) == INF:
                assert np.isinf(d[i]) and (d[i] < 0) == (want < 0)
                continue
            assert F(d[i]) == want
            assert bool(np.signbit(d[i])) == bool(c & 8)


def test_roundtrip_error_bound():
    # |x - deq| <= half the grid spacing at x's magnitude, times the block scale
    x = workloads.mxfp4_weight(8, 256, seed=15, dtype=torch.float32).numpy()
    packed, e8m0 = mx.quantize(x)
    d = mx.dequantize(packed, e8m0, 256)
    sc = np.repeat(np.ldexp(1.0, e8m0.astype(np.int32) - 127), 32, axis=1)
    v = np.abs(x) / sc
    spacing = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
    err = np.abs(x - d) / sc
    assert np.all(err <= spacing / 2 + (v > 6) * (v - 6))
