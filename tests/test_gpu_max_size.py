"""Oracle parity at the largest weight the library takes: N * K just below 2^31 elements.

The boundary refuses N * K >= 2^31 (tests/test_boundary.py); here a bf16 weight of
131064 x 16384 = 2^31 - 131072 elements (the width of a large model's vocabulary head)
goes through the benchmark's calls, gwb_quantize_snr then gwb_dequantize to bf16, for
MXFP4 (page quantize_dflash_mxfp4.py), GPTQ symmetric g128 (page export_gptq_cpu.py) and
uintx4 g64 (page uintx_quant.py), so every element, unit, tile and shard index runs up to
the top of its range. Rows spread over the whole matrix, first and last included, are
checked bit for bit against the oracle (for uintx every shard byte that holds one of
them); the fused reconstruction sums against float64 sums of the whole matrix (W itself,
and W minus the dequantized values the sums are defined on: bf16 for MXFP4 and uintx,
float32 (c - 8) * s for GPTQ, whose sampled rows matched the oracle), within the fused
pass's bound. The weight is drawn on the device (seeded): N(0, 0.015) times a
per-row gain lognormal(0, 0.5), the metric workload's recipe at this size.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.gptq as ogq
import oracle.mxfp4 as omx
import oracle.uintx as oux
from oracle._fp import bf16_round

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from group_wise_bit_amd import binding as gwb      # must load: no fallback where a GPU is present
else:  # collected on CPU only to be skipped
    gwb = None

DEV = "cuda"
N, K = 131064, 16384
FUSED_REL = 72 * 2.0 ** -24 + 1e-12     # the fused pass's float32 sums of up to 64 terms per lane, relative


def _np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def _bf16bits(t: torch.Tensor) -> np.ndarray:
    return _np(t.contiguous().view(torch.int16)).view(np.uint16)


def _ref_bf16bits(x) -> np.ndarray:
    return (np.asarray(bf16_round(x), np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _draw(n, k, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    W = torch.empty(n, k, dtype=torch.bfloat16, device=DEV)
    gain = torch.exp(0.5 * torch.randn(n, generator=g, device=DEV))
    for r0 in range(0, n, 8192):                   # float32 draws in row bands, rounded to bf16
        r1 = min(n, r0 + 8192)
        band = torch.randn(r1 - r0, k, generator=g, device=DEV) * 0.015 * gain[r0:r1, None]
        W[r0:r1] = band.to(torch.bfloat16)
    return W


@pytest.fixture(scope="module")
def big_weight():
    assert N * K < 2 ** 31 and (2 ** 31 - N * K) == 131072
    W = _draw(N, K, 2031)
    yield W
    del W
    torch.cuda.empty_cache()


def _rows(count, seed, mult=1):
    r = np.random.default_rng(seed).choice(N // mult, count, replace=False) * mult
    return np.unique(np.concatenate([r, [0, N - mult]]))


def _sums(W: torch.Tensor, D: torch.Tensor):
    """float64 sum of w^2 and of (w - d)^2 over the whole matrix, in row bands."""
    sw = se = 0.0
    for r0 in range(0, W.shape[0], 8192):
        w = W[r0:r0 + 8192].double()
        sw += float((w * w).sum())
        e = w - D[r0:r0 + 8192].double()
        se += float((e * e).sum())
    return sw, se


def _check_sums(snr: torch.Tensor, W, D):
    sw, se = _sums(W, D)
    got = _np(snr)
    assert got[0] == pytest.approx(sw, rel=FUSED_REL)
    assert got[1] == pytest.approx(se, rel=FUSED_REL)


def test_max_size_mxfp4(big_weight):
    W = big_weight
    q, snr = gwb.quantize_snr(W, "mxfp4")
    d = gwb.dequantize(q, torch.bfloat16)
    rows = _rows(40, 31)
    w = W[rows].float().cpu().numpy()
    p, e = omx.quantize(w)
    assert np.array_equal(_np(q["packed"][rows]), p)
    assert np.array_equal(_np(q["e8m0"][rows]), e)
    assert np.array_equal(_bf16bits(d[rows]), _ref_bf16bits(omx.dequantize(p, e, K)))
    _check_sums(snr, W, d)
    del q, d
    torch.cuda.empty_cache()


def test_max_size_gptq_sym(big_weight):
    W = big_weight
    q, snr = gwb.quantize_snr(W, "gptq_sym", group=128)
    d = gwb.dequantize(q, torch.bfloat16)
    bands = _rows(12, 32, mult=8)                  # whole 8-row bands: one qzeros word each
    rows = np.concatenate([np.arange(b, b + 8) for b in bands])
    o = ogq.quantize_sym(W[rows].float().cpu().numpy(), 128)
    qw = _np(q["qweight"])
    assert np.array_equal(qw[:, rows], o["qweight"])
    assert np.array_equal(_np(q["scales"])[:, rows], o["scales"])
    assert np.array_equal(_np(q["qzeros"])[:, bands // 8], o["qzeros"])
    ref = ogq.dequantize(o["qweight"], o["scales"], o["qzeros"], 128, True)
    assert np.array_equal(_bf16bits(d[rows]), _ref_bf16bits(ref))
    del d
    d32 = gwb.dequantize(q, torch.float32)        # the fused sums use the exact (c - 8) * s
    assert np.array_equal(_np(d32[rows]), ref)
    _check_sums(snr, W, d32)
    del q, d32
    torch.cuda.empty_cache()


def test_max_size_uintx4(big_weight):
    W = big_weight
    nbits = 4
    q, snr = gwb.quantize_snr(W, "uintx", nbits=nbits)
    d = gwb.dequantize(q, torch.bfloat16)
    packed = q["packed"]
    numel = N * K
    rng = np.random.default_rng(33)
    plan, need_rows, base, off = [], set(), 0, 0
    for kb in oux.shard_widths(nbits):
        L = oux.shard_nbytes(numel, kb)
        idx = np.concatenate([rng.choice(L, 24, replace=False), [0, L - 1]])
        for i in idx:
            elems = [j * L + int(i) for j in range(8 // kb)]
            need_rows.update(e // K for e in elems)
            plan.append((base + int(i), kb, off, elems))
        base += L
        off += kb
    rows = np.array(sorted(need_rows))
    o = oux.quantize(W[rows].float().cpu().numpy(), nbits)
    pos = {int(r): p for p, r in enumerate(rows)}
    got = _np(packed[torch.tensor([b for b, _, _, _ in plan], device=DEV)])
    for (byte_at, kb, sh, elems), gb in zip(plan, got):
        v = 0
        for j, e in enumerate(elems):
            c = int(o["codes"][pos[e // K], e % K])
            v |= ((c >> sh) & ((1 << kb) - 1)) << (j * kb)
        assert int(gb) == v, byte_at
    assert np.array_equal(_np(q["scale_bytes"][rows]), o["scale_bytes"])
    assert np.array_equal(_np(q["zero_point"][rows]), o["zero_point"])
    ref = oux.dequantize(o["packed"], o["scale_bytes"], o["zero_point"], nbits, len(rows), K)
    assert np.array_equal(_bf16bits(d[rows]), _ref_bf16bits(ref))
    _check_sums(snr, W, d)
    del q, d
    torch.cuda.empty_cache()


def test_max_size_mxfp4_row_bands():
    """MXFP4 past 2^31 elements: 131080 x 16384 = 2^31 + 131072 runs as row bands of
    131071 and 9 rows (each under the kernels' 32-bit indices). Rows on both sides of the
    band edge and spread over the matrix bit for bit against the oracle; the fused sums
    and gwb_snr's (every band's partials in one finalize) against float64 sums of the
    whole matrix."""
    n = 131080
    assert n * K >= 2 ** 31 and (2 ** 31 - 1) // K == 131071
    W = _draw(n, K, 2032)
    q, snr = gwb.quantize_snr(W, "mxfp4")
    d = gwb.dequantize(q, torch.bfloat16)
    rows = np.unique(np.concatenate([np.random.default_rng(34).choice(n, 40, replace=False),
                                     [0, 131069, 131070, 131071, 131072, n - 1]]))
    w = W[rows].float().cpu().numpy()
    p, e = omx.quantize(w)
    assert np.array_equal(_np(q["packed"][rows]), p)
    assert np.array_equal(_np(q["e8m0"][rows]), e)
    assert np.array_equal(_bf16bits(d[rows]), _ref_bf16bits(omx.dequantize(p, e, K)))
    _check_sums(snr, W, d)
    s2 = gwb.snr(W, q)
    _check_sums(s2, W, d)
    del q, d, W
    torch.cuda.empty_cache()
