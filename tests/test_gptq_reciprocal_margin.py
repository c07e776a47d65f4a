"""CPU proof by exhaustion of the GPTQ quantize kernel's reciprocal shortcut.

The kernel (group_wise_bit_amd/csrc/gptq.hip, gptq_quant_kernel) forms a code as
rint(u) with u = fma(x, y, zp), y the hardware reciprocal of the float32 scale s
(v_rcp_f32: within 1 ulp of 1/s), and keeps it when |u - rint(u)| is below
margin = 0.5 - fma(a, y, 16) * 2^-19 (a the group's largest magnitude); any other weight
is divided exactly. Page export_gptq_cpu.py (quantize_sym / quantize_asym) defines the
code as rint(x / s) + zp with an IEEE float32 quotient. This test models every float32 y
within one ulp of 1/s (the float32 neighbours of 1/s and the nearest one's neighbours),
evaluates each fma and subtraction with one float32 rounding exactly as the kernel does,
and checks that every accepted code equals rint(fl(x / s)) + zp: over every bf16 weight
of many groups (random and adversarial extremes, symmetric and asymmetric scales, exact
and near ties) and over random float32 groups. A planted margin without the error
allowance must fail it.
"""
import numpy as np

F32, F64 = np.float32, np.float64


def _fma32(a, b, c):
    """float32(a * b + c) with one rounding: the product is exact in float64; the sum's
    float64 rounding error is recovered (two-sum) and decides float32 ties."""
    p = a.astype(F64) * b.astype(F64)
    c64 = c.astype(F64)
    s = p + c64
    bb = s - p
    err = (p - (s - bb)) + (c64 - bb)
    r = s.astype(F32)
    r64 = r.astype(F64)
    other = np.where(r64 > s, np.nextafter(r, F32(-np.inf)), np.nextafter(r, F32(np.inf)))
    mid = (r64 + other.astype(F64)) / 2
    fix = (s == mid) & (err != 0)
    up = np.maximum(r, other)
    dn = np.minimum(r, other)
    return np.where(fix, np.where(err > 0, up, dn), r).astype(F32)


def _recips(s):
    """Every float32 within one ulp of 1/s (a superset: RN(1/s) and its neighbours)."""
    y = (F64(1.0) / s.astype(F64)).astype(F32)
    return [np.nextafter(y, F32(-np.inf)), y, np.nextafter(y, F32(np.inf))]


def _check(x, s, zp, a, allowance=True):
    """x: float32 weights of one group (array); s, zp, a: float32 scalars.
    Returns (accepted count, mismatches among accepted)."""
    exact = np.rint((x / s).astype(F32)) + zp                   # IEEE float32 quotient
    acc, bad = 0, 0
    for y in _recips(np.array([s], F32)):
        yv = np.full_like(x, y[0])
        u = _fma32(x, yv, np.full_like(x, zp))
        c = np.rint(u)
        dev = np.abs(u - c)                                      # exact (Sterbenz)
        t = _fma32(np.array([a], F32), y, np.array([16.0], F32))[0]
        margin = F32(0.5) - F32(t * F32(2.0 ** -19)) if allowance else F32(0.5)
        if not margin > 0:
            continue                                             # the kernel divides every weight
        ok = dev < margin
        acc += int(ok.sum())
        bad += int((c[ok] != exact[ok]).sum())
    return acc, bad


def _all_bf16():
    b = np.arange(65536, dtype=np.uint32) << 16
    v = b.view(F32)
    return v[np.isfinite(v)]


def _groups(rng, n):
    """(amax or (mn, mx)) draws over many binades, with exact half-step maxima."""
    e = rng.integers(-30, 30, n)
    m = rng.integers(128, 256, n)                               # bf16 significands
    return (m.astype(F64) * 2.0 ** (e - 7)).astype(F32)


def test_sym_shortcut_every_bf16_weight():
    rng = np.random.default_rng(11)
    xs = _all_bf16()
    total = 0
    for amax in _groups(rng, 120):
        s = max(F32(amax * F32(0.125)), F32(1e-9))
        x = xs[np.abs(xs) <= amax]
        acc, bad = _check(x, s, F32(8.0), amax)
        assert bad == 0, (amax, s)
        total += acc
    assert total > 0


def test_asym_shortcut_every_bf16_weight():
    rng = np.random.default_rng(12)
    xs = _all_bf16()
    lo, hi = _groups(rng, 120), _groups(rng, 120)
    for i in range(120):
        mn, mx = -lo[i] if i % 3 else F32(0.0), hi[i]
        if i % 5 == 0:                                          # groups away from zero
            mn, mx = hi[i] * F32(0.5), hi[i]
        s = F32(max(F32(mx - mn), F32(1e-9)) / F32(15.0))
        zp = F32(np.clip(np.rint(F32(-mn / s)), 0, 15))
        a = max(abs(mn), abs(mx))
        x = xs[(xs >= mn) & (xs <= mx)]
        acc, bad = _check(x, s, zp, F32(a))
        assert bad == 0, (mn, mx, s, zp)


def test_shortcut_exact_ties_and_float32_weights():
    rng = np.random.default_rng(13)
    for _ in range(200):
        amax = _groups(rng, 1)[0]
        s = F32(amax * F32(0.125))
        k = rng.integers(-16, 17, 4096).astype(F64) / 2           # every half step: exact ties
        near = (k * s).astype(F32)
        x = np.concatenate([near, np.nextafter(near, F32(np.inf)), np.nextafter(near, F32(-np.inf)),
                            (rng.uniform(-1, 1, 4096) * amax).astype(F32)])
        x = x[np.abs(x) <= amax]
        acc, bad = _check(x, s, F32(8.0), amax)
        assert bad == 0


def test_shortcut_accepts_almost_everything():
    """The shortcut is worth having: all but a small fraction of weights are accepted."""
    rng = np.random.default_rng(14)
    xs = _all_bf16()
    acc_all, n_all = 0, 0
    for amax in _groups(rng, 20):
        x = xs[np.abs(xs) <= amax]
        acc, _ = _check(x, F32(amax * F32(0.125)), F32(8.0), amax)
        acc_all += acc
        n_all += 3 * x.size
    assert acc_all > 0.98 * n_all


def test_margin_without_error_allowance_fails():
    """Planted mistake: accepting whenever |u - rint(u)| < 0.5 (no allowance for the
    reciprocal's error) gives wrong codes near ties."""
    rng = np.random.default_rng(15)
    bad_total = 0
    for _ in range(60):
        amax = _groups(rng, 1)[0]
        s = F32(amax * F32(0.125))
        k = rng.integers(-16, 17, 4096).astype(F64) / 2
        near = (k * s).astype(F32)
        x = np.concatenate([near, np.nextafter(near, F32(np.inf)), np.nextafter(near, F32(-np.inf))])
        x = x[np.abs(x) <= amax]
        bad_total += _check(x, s, F32(8.0), amax, allowance=False)[1]
    assert bad_total > 0


def test_fma32_emulation_is_one_rounding():
    """The float32 fma model against exact rational arithmetic (tests/_exact.py)."""
    from _exact import F, rn32
    rng = np.random.default_rng(16)
    a = (rng.standard_normal(3000) * 2.0 ** rng.integers(-40, 40, 3000)).astype(F32)
    b = (rng.standard_normal(3000) * 2.0 ** rng.integers(-40, 40, 3000)).astype(F32)
    c = (rng.integers(0, 16, 3000)).astype(F32)
    c[::3] = (-(a[::3].astype(F64) * b[::3].astype(F64))).astype(F32)      # heavy cancellation
    got = _fma32(a, b, c)
    for i in range(3000):
        assert F(got[i]) == rn32(F(a[i]) * F(b[i]) + F(c[i])), i


def _sym_tie_rule(x, amax, recips_all=True, rule=np.rint):
    """The kernel's symmetric bf16 path for weights that fail the margin: h = rint(u) +-
    1/2 towards u, code rint(h). Returns (rejected count, mismatches, non-ties among the
    rejected) against the page's rint(fl(x / s)) + 8."""
    s = F32(amax * F32(0.125))
    exact = np.rint((x / s).astype(F32)) + F32(8.0)
    rej, bad, nontie = 0, 0, 0
    ys = _recips(np.array([s], F32)) if recips_all else [np.array([(F64(1.0) / F64(s))], F32)]
    for y in ys:
        u = _fma32(x, np.full_like(x, y[0]), np.full_like(x, F32(8.0)))
        c = np.rint(u)
        t = _fma32(np.array([amax], F32), y, np.array([16.0], F32))[0]
        margin = F32(0.5) - F32(t * F32(2.0 ** -19))
        fail = ~(np.abs(u - c) < margin)
        if not fail.any():
            continue
        xf = x[fail].astype(F64)
        m = np.rint(16.0 * xf / F64(amax))                      # 2 x / s, an odd integer at a tie
        nontie += int(((16.0 * xf != m * F64(amax)) | (m % 2 == 0)).sum())
        h = c[fail] + np.copysign(F32(0.5), u[fail] - c[fail])
        code = rule(h).astype(F32)
        rej += int(fail.sum())
        bad += int((code != exact[fail]).sum())
    return rej, bad, nontie


def test_sym_bf16_margin_failures_are_exact_ties():
    """Symmetric groups of bf16 weights (s = amax / 8, exact): every weight that fails the
    margin is an exact tie x / s = k + 1/2, and the kernel's rint(h) equals the page's
    rint(fl(x / s)) + 8 - over every bf16 weight of 240 groups, every reciprocal within
    one ulp, and every significand pair of an amax and a weight."""
    rng = np.random.default_rng(17)
    xs = _all_bf16()
    rej_total = 0
    for amax in _groups(rng, 240):
        if amax * F32(0.125) < F32(1e-9):
            continue
        x = xs[np.abs(xs) <= amax]
        rej, bad, nontie = _sym_tie_rule(x, amax)
        assert bad == 0 and nontie == 0, (amax, bad, nontie)
        rej_total += rej
    assert rej_total > 0
    # every pair of significands (the quotient depends on them and the exponent gap)
    mx = np.arange(128, 256, dtype=F64)
    for ma in range(128, 256):
        amax = F32(ma)
        for gap in range(0, 12):
            x = np.concatenate([mx, -mx]) * 2.0 ** (-gap - 1)
            x = x.astype(F32)
            x = x[np.abs(x) <= amax]
            rej, bad, nontie = _sym_tie_rule(x, amax, recips_all=False)
            assert bad == 0 and nontie == 0, (ma, gap)


def test_sym_tie_rule_needs_round_half_even():
    """Planted mistake: rounding the half step away from zero instead of to even."""
    rng = np.random.default_rng(18)
    xs = _all_bf16()
    away = lambda h: np.sign(h) * np.floor(np.abs(h) + 0.5)
    bad_total = 0
    for amax in _groups(rng, 60):
        x = xs[np.abs(xs) <= amax]
        bad_total += _sym_tie_rule(x, amax, rule=away)[1]
    assert bad_total > 0
