"""Pins for the affine uintx oracle (page uintx_quant.py: _pack_shard, _unpack_shard,
pack_uintx, unpack_uintx, UIntXQuantizer.can_quantize/_quantize_impl/_dequantize_native)."""
import numpy as np
import pytest
import torch

import oracle.uintx as ux
from _exact import INF, F, rint_even, rn32, rnbf16, rnf16, same
from golden.golden import floats, hexbytes, load
from group_wise_bit_amd import workloads

EPS = F(np.float32(2.0 ** -23))


def test_pack_worked_examples():
    g = load("uintx_pack_examples.txt")
    for key, val in g.items():
        nbits = int(key[4:])
        codes_s, bytes_s = val.split("=>")
        codes = np.array([int(t) for t in codes_s.split()], np.uint8)
        want = b"".join(hexbytes(part) for part in bytes_s.split("|"))
        got = ux.pack(codes, nbits)
        assert got.tobytes() == want, key
        assert np.array_equal(ux.unpack(got, nbits, codes.size), codes)


@pytest.mark.parametrize("nbits", [2, 3, 4, 5, 6, 7])
@pytest.mark.parametrize("numel", [1, 5, 8, 63, 64, 100, 512, 1000, 4096])
def test_pack_roundtrip_and_sizes(nbits, numel):
    rng = np.random.default_rng(nbits * 1000 + numel)
    c = rng.integers(0, 1 << nbits, numel).astype(np.uint8)
    p = ux.pack(c, nbits)
    assert p.size == ux.packed_nbytes(numel, nbits)
    if numel % 8 == 0:
        assert p.size == numel * nbits // 8
    assert np.array_equal(ux.unpack(p, nbits, numel), c)


def test_shard_order_low_bits_in_widest_shard():
    # nbits 7 = 4 + 2 + 1: the 4-bit shard holds bits 0..3, the 2-bit shard bits 4..5
    c = np.array([0b1011010] * 8, np.uint8)
    p = ux.pack(c, 7)
    assert p[:4].tolist() == [0b10101010] * 4      # low nibble 1010 twice per byte
    assert p[4:6].tolist() == [0b01010101] * 2     # bits 4..5 = 01 four times per byte
    assert p[6] == 0b11111111                      # bit 6 set in all eight


def test_worked_example_group():
    g = load("uintx_worked_group.txt")
    w = np.zeros((1, 64), np.float32)
    head = floats(g["w_head"])
    w[0, :len(head)] = head
    q = ux.quantize(w, 2)
    assert q["codes"][0, :5].tolist() == [int(t) for t in g["codes_head"].split()]
    assert q["packed"].tobytes() == hexbytes(g["packed_hex"])
    assert q["scale_bytes"].tobytes() == hexbytes(g["scale_bytes_hex"])
    assert q["zero_point"].tolist() == [[int(g["zero_point"])]]
    d = ux.dequantize(q["packed"], q["scale_bytes"], q["zero_point"], 2, 1, 64)
    assert d[0, :5].tolist() == floats(g["dequant_head"])


def _exact_group(xs, nbits, rn=rnbf16):
    """Each op of the weight dtype as an exact result rounded once to that dtype (rn).
    An infinite float16 reciprocal sends positive weights to qmax and the rest to 0
    (zeros: the NaN of 0 * inf, converted to code 0)."""
    qmax = (1 << nbits) - 1
    mn = min(min(F(v) for v in xs), F(0))
    mx = max(max(F(v) for v in xs), F(0))
    s = rn(rn(mx - mn) / qmax)
    s = max(s, EPS)
    zp = min(max(-rint_even(rn(mn / s)), 0), qmax)
    inv = rn(1 / s)
    codes = []
    for v in xs:
        if inv == INF:
            codes.append(qmax if F(v) > 0 else 0)
            continue
        t = rn(F(v) * inv)
        if t in (INF, -INF):
            codes.append(qmax if t > 0 else 0)
            continue
        r = rint_even(t) + zp                      # integers: the rounded add only matters
        codes.append(min(max(r, 0), qmax))         # beyond the clamp
    return s, zp, codes


@pytest.mark.parametrize("nbits", [2, 3, 5, 7])
def test_quantize_bruteforce_exact(nbits):
    ws = [workloads.uintx_weight(4, 256, seed=31).float().numpy(),
          workloads.adversarial_weight(8, 256, seed=32, dtype=torch.bfloat16).float().numpy()]
    for w in ws:
        q = ux.quantize(w, nbits)
        n, k = w.shape
        for r in range(n):
            for g in range(k // 64):
                xs = w[r, 64 * g:64 * g + 64]
                s, zp, codes = _exact_group(xs.tolist(), nbits)
                assert same(q["scale"][r, g], s)
                assert q["zero_point"][r, g] == zp
                assert q["codes"][r, 64 * g:64 * g + 64].tolist() == codes


def test_double_rounding_is_exercised():
    # bf16(w * inv) then rint differs from rint of the exact product on some inputs
    w = workloads.uintx_weight(64, 1024, seed=33).float().numpy()
    q = ux.quantize(w, 4)
    inv = np.repeat(np.array([[float(rnbf16(1 / F(s))) for s in row] for row in q["scale"]], np.float64), 64, 1)
    exact = w.astype(np.float64) * inv
    bf = np.array([float(rnbf16(F(v))) for v in exact.ravel()[:200000]])
    n_diff = int(np.sum(np.rint(bf) != np.rint(exact.ravel()[:200000])))
    assert n_diff > 0


@pytest.mark.parametrize("nbits", [2, 3, 4, 5, 6, 7])
def test_preserve_zero_and_ranges(nbits):
    w = workloads.uintx_weight(32, 512, seed=34).float().numpy()
    w[:, ::7] = 0.0
    q = ux.quantize(w, nbits)
    assert q["zero_point"].max() <= (1 << nbits) - 1
    assert q["codes"].max() <= (1 << nbits) - 1
    d = ux.dequantize(q["packed"], q["scale_bytes"], q["zero_point"], nbits, 32, 512)
    assert np.all(d[:, ::7] == 0.0)
    assert np.array_equal(ux.unpack(q["packed"], nbits, w.size).reshape(w.shape), q["codes"])


def test_dequant_exact():
    w = workloads.adversarial_weight(4, 256, seed=35, dtype=torch.bfloat16).float().numpy()
    q = ux.quantize(w, 5)
    d = ux.dequantize(q["packed"], q["scale_bytes"], q["zero_point"], 5, 4, 256)
    for r in range(4):
        for k in range(256):
            c, z = int(q["codes"][r, k]), int(q["zero_point"][r, k // 64])
            assert same(d[r, k], rnbf16((c - z) * F(q["scale"][r, k // 64])))


def test_can_quantize_refusals():
    assert not ux.can_quantize(8, (64, 128))
    assert not ux.can_quantize(4, (64, 100))
    assert not ux.can_quantize(4, (2, 64, 128))
    assert ux.can_quantize(7, (64, 128))


def test_bits_per_weight():
    assert ux.bits_per_weight(4) == 4.375


def test_reading_division_vs_reciprocal_identical_after_bf16():
    # torch evaluates bf16 / python-scalar as a division on the CPU and as a multiply by
    # the float32 reciprocal on the GPU; after the bf16 rounding both agree for every
    # positive finite bf16 and every qmax used here, so the scale is well defined.
    u = np.arange(1, 0x7F80, dtype=np.uint32)
    x = (u << 16).view(np.float32)
    for qmax in (3, 7, 15, 31, 63, 127):
        a = ux.bf(x / np.float32(qmax))
        b = ux.bf(x * (np.float32(1.0) / np.float32(qmax)))
        assert np.array_equal(a, b), qmax


RN = {"f16": rnf16, "f32": rn32}
TDT = {"f16": torch.float16, "f32": torch.float32}


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("nbits,group", [(2, 32), (4, 64), (3, 128), (7, 64)])
def test_quantize_bruteforce_exact_other_dtypes(dtype, nbits, group):
    """float16 / float32 weights: every op one rounding to the weight dtype (float32:
    IEEE division), any group size dividing K."""
    ws = [workloads.uintx_weight(4, 256, seed=36, dtype=TDT[dtype]).float().numpy(),
          workloads.adversarial_weight(6, 256, seed=37, dtype=TDT[dtype]).float().numpy()]
    for w in ws:
        q = ux.quantize(w, nbits, group, dtype)
        n, k = w.shape
        for r in range(n):
            for g in range(k // group):
                xs = w[r, group * g:group * (g + 1)]
                s, zp, codes = _exact_group(xs.tolist(), nbits, RN[dtype])
                assert same(q["scale"][r, g], s), (r, g)
                assert q["zero_point"][r, g] == zp
                assert q["codes"][r, group * g:group * (g + 1)].tolist() == codes, (r, g)


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_dequant_exact_other_dtypes(dtype):
    w = workloads.adversarial_weight(4, 256, seed=38, dtype=TDT[dtype]).float().numpy()
    q = ux.quantize(w, 5, 32, dtype)
    assert q["scale_bytes"].shape == (4, 8 * ux.SCALE_BYTES[dtype])
    d = ux.dequantize(q["packed"], q["scale_bytes"], q["zero_point"], 5, 4, 256, 32, dtype)
    for r in range(4):
        for k in range(256):
            c, z = int(q["codes"][r, k]), int(q["zero_point"][r, k // 32])
            assert same(d[r, k], RN[dtype]((c - z) * F(q["scale"][r, k // 32])))


def test_float16_infinite_reciprocal_group():
    """Hand-worked float16 group, nbits 4: 62 weights 2**-20, one 0, one -2**-22.
    Range 5 * 2**-22, / 15 = (4/3) 2**-24 rounds to the subnormal 2**-24, clamped to
    2**-23 (float16 bits 0x0002); zp = -rint(-2**-22 / 2**-23) = 2; 1 / 2**-23 overflows
    float16 to inf, so the positives take 15, the negative 0 and the zero 0 (NaN)."""
    w = np.full((1, 64), 2.0 ** -20, np.float32)
    w[0, 3] = 0.0
    w[0, 5] = -(2.0 ** -22)
    q = ux.quantize(w, 4, 64, "f16")
    want = [15] * 64
    want[3] = 0
    want[5] = 0
    assert q["codes"][0].tolist() == want
    assert q["zero_point"].tolist() == [[2]]
    assert q["scale_bytes"].tobytes() == bytes([0x02, 0x00])
    d = ux.dequantize(q["packed"], q["scale_bytes"], q["zero_point"], 4, 1, 64, 64, "f16")
    assert d[0, 0] == 13 * 2.0 ** -23 and d[0, 3] == -(2.0 ** -22)


def test_reading_division_vs_reciprocal_identical_after_f16():
    # float16 counterpart of the bf16 check: every positive finite float16.
    x = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    for qmax in (3, 7, 15, 31, 63, 127):
        a = ux.f16(x / np.float32(qmax))
        b = ux.f16(x * (np.float32(1.0) / np.float32(qmax)))
        assert np.array_equal(a, b), qmax


def test_reading_float32_division_is_ieee():
    # float32 weights: the scale is the correctly rounded quotient, which a multiply by
    # the float32 reciprocal misses for some ranges (here 0.3 over qmax 3).
    w = np.zeros((1, 64), np.float32)
    w[0, 0] = np.float32(0.3)
    q = ux.quantize(w, 2, 64, "f32")
    assert same(q["scale"][0, 0], rn32(F(np.float32(0.3)) / 3))
    assert q["scale"][0, 0] != np.float32(0.3) * (np.float32(1.0) / np.float32(3.0))


def test_bits_per_weight_other_dtypes():
    assert ux.bits_per_weight(4, 64, "f16") == 4.375
    assert ux.bits_per_weight(4, 32, "f32") == 5.25
