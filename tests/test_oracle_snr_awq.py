"""Pins for the SNR oracle (page export_gptq_cpu.py's in-function SNR; page
quantize_dflash_mxfp4.py's relative error) and the AWQ alpha search (page
quantize_dflash_mxfp4.py, search_scale and the diagonal surrogate in its docstring)."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.awq as awq
import oracle.snr as snr
from _exact import F, mxfp4_block_exact, mxfp4_dequant_exact, rn32
from group_wise_bit_amd import workloads


def test_snr_closed_form_relative_perturbation():
    rng = np.random.default_rng(41)
    w = (rng.integers(-2 ** 12, 2 ** 12, (64, 64)) * 2.0 ** -14).astype(np.float32)
    for k in (4, 8, 12):
        d = (w * np.float32(1 + 2.0 ** -k)).astype(np.float32)   # exact: few mantissa bits
        assert np.all(w.astype(np.float64) * (1 + 2.0 ** -k) == d)
        assert snr.snr_db(w, d) == pytest.approx(20 * k * math.log10(2), abs=1e-9)
        sw, se = snr.sums(w, d)
        assert snr.rel_error(sw, se) == pytest.approx(2.0 ** -k, rel=1e-12)


def test_snr_identical_and_zero():
    w = np.linspace(-1, 1, 256, dtype=np.float32)
    s = float(np.sum(w.astype(np.float64) ** 2))
    assert snr.snr_db(w, w) == pytest.approx(10 * math.log10(s / 1e-24))
    assert snr.snr_db(np.zeros(8, np.float32), np.zeros(8, np.float32)) == -math.inf


def test_snr_matches_norm_form():
    rng = np.random.default_rng(42)
    w = rng.standard_normal(1000).astype(np.float32)
    d = (w + rng.standard_normal(1000).astype(np.float32) * np.float32(0.01)).astype(np.float32)
    num = math.sqrt(math.fsum(float(v) ** 2 for v in w))
    den = math.sqrt(math.fsum(float(v) ** 2 for v in (w - d)))
    assert snr.snr_db(w, d) == pytest.approx(20 * math.log10(num / den), abs=1e-9)


def test_subsample_rows_of_gate_up_shape():
    idx = np.arange(34816)[:, None]
    sub = awq.subsample_rows(idx, 2048)
    assert sub.shape == (2048, 1)
    assert sub[0, 0] == 0 and sub[1, 0] == 17 and sub[-1, 0] == 34799
    small = np.arange(100)[:, None]
    assert np.array_equal(awq.subsample_rows(small, 2048), small)
    odd = awq.subsample_rows(np.arange(5000)[:, None], 2048)   # stride 2 -> 2500 rows, keep 2048
    assert odd.shape[0] == 2048 and odd[-1, 0] == 4094


def test_scale_table_properties():
    a = workloads.awq_activation_stat(512, seed=43).numpy()
    t = awq.scale_table(a)
    assert np.all(t[0] == 1.0)                                  # alpha = 0 -> s == 1 exactly
    for row in t:
        g = math.exp(math.fsum(math.log(float(v)) for v in row) / row.size)
        assert abs(g - 1) < 1e-6                                # geometric mean 1 (float32 rounding)
        assert np.all(row > 0)
    # clamp: an**1 spans far beyond [1e-2, 1e2] for lognormal(0, 1) at this size?
    an = a.astype(np.float64) / a.astype(np.float64).mean()
    ref = np.clip(an, 1e-2, 1e2)
    ref = ref / np.exp(np.mean(np.log(ref)))
    assert np.allclose(t[-1], ref, rtol=1e-7, atol=0)


def test_constant_stat_gives_identity_scaling_and_alpha_zero():
    w = workloads.mxfp4_weight(64, 256, seed=44, dtype=torch.float32).numpy()
    a = np.full(256, 0.37, np.float32)
    r = awq.search(w, a)
    assert np.all(r["s_table"] == 1.0)
    assert np.all(r["errors"] == r["errors"][0])
    assert r["best"] == 0                                       # strict < keeps the first


def _exact_error(W, a, s):
    """The surrogate error with every float32 op rounded exactly once."""
    n, k = W.shape
    a = [max(F(v), F(np.float32(1e-8))) for v in a]
    total = Fraction(0)
    for r in range(n):
        X = [rn32(F(W[r, j]) * F(s[j])) for j in range(k)]
        for b in range(k // 32):
            blk = [float(v) for v in X[32 * b:32 * b + 32]]
            codes, e = mxfp4_block_exact(blk)
            for i, c in enumerate(codes):
                j = 32 * b + i
                D = mxfp4_dequant_exact(c, e + 127)
                q = rn32(D / F(s[j]))
                t = rn32(rn32(q - F(W[r, j])) * a[j])
                total += rn32(t * t)
    return total


def test_weighted_error_bruteforce_exact():
    W = workloads.mxfp4_weight(6, 64, seed=45, dtype=torch.bfloat16).float().numpy()
    a = workloads.awq_activation_stat(64, seed=46).numpy()
    t = awq.scale_table(a)
    for i in (0, 3, 7, 10):
        got = awq.weighted_error(W, a, t[i])
        want = float(_exact_error(W, a, t[i]))
        assert got == pytest.approx(want, rel=1e-12)


def test_search_picks_minimum():
    W = workloads.mxfp4_weight(256, 512, seed=47, dtype=torch.bfloat16).float().numpy()
    a = workloads.awq_activation_stat(512, seed=48).numpy()
    r = awq.search(W, a)
    assert r["best"] == int(np.argmin(r["errors"]))
    assert r["best_alpha"] == r["best"] / 10
