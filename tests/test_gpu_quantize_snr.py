"""GPU checks of gwb_quantize_snr, quantization and SNR in one pass over W: the stored
tensors equal gwb_quantize's bit for bit, and the three SNR values equal gwb_snr's (the
fused sums differ only in float64 summation order) and the float64 sums over the
dequantized matrix on the host (page export_gptq_cpu.py's 20 log10(||w|| / ||w - deq||)
of the stored values, as gwb_snr defines it)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from group_wise_bit_amd import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from group_wise_bit_amd import binding as gwb      # must load: no fallback on a GPU machine
else:  # collected on CPU only to be skipped
    gwb = None

DEV = "cuda"
_TDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _host_sums(W, q):
    d = gwb.dequantize(q, q.w_dtype if q.fmt == "uintx" else torch.float32).float().cpu().double()
    w = W.float().cpu().double()
    e = (W.float().cpu() - d.float()).double()
    return float((w * w).sum()), float((e * e).sum())


def _check(W, fmt, nbits=4, group=None):
    Wd = W.to(DEV)
    q1 = gwb.quantize(Wd, fmt, nbits=nbits, group=group)
    s1 = gwb.snr(Wd, q1).cpu().numpy()
    q2, s2 = gwb.quantize_snr(Wd, fmt, nbits=nbits, group=group)
    s2 = s2.cpu().numpy()
    assert torch.equal(q1.codes, q2.codes) and torch.equal(q1.scales, q2.scales)
    if q1.zeros is not None:
        assert torch.equal(q1.zeros, q2.zeros)
    assert s2[0] == pytest.approx(s1[0], rel=1e-12) and s2[1] == pytest.approx(s1[1], rel=1e-12, abs=1e-300)
    assert s2[2] == pytest.approx(s1[2], rel=1e-10, abs=1e-9)
    w2, e2 = _host_sums(W, q2)
    assert s2[0] == pytest.approx(w2, rel=1e-9) and s2[1] == pytest.approx(e2, rel=1e-9, abs=1e-300)
    return s1, s2


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp4_page_ties"])
@pytest.mark.parametrize("n,k,ld", [(64, 512, 512), (37, 96, 96), (130, 2048, 2080)])
def test_quantize_snr_mxfp4(fmt, n, k, ld):
    """MXFP4 runs the error kernel's grid and per-thread order: the sums are bit-identical
    to gwb_snr's (row strides too)."""
    Wf = workloads.mxfp4_weight(n, ld, seed=800 + n)
    W = Wf[:, :k]
    s1, s2 = _check(W, fmt)
    assert np.array_equal(s1[:2], s2[:2])


@pytest.mark.parametrize("fmt", ["gptq_sym", "gptq_asym"])
@pytest.mark.parametrize("group", [32, 64, 128])
@pytest.mark.parametrize("n,k", [(64, 512), (72, 640), (264, 1536)])
def test_quantize_snr_gptq(fmt, group, n, k):
    W = workloads.mxfp4_weight(n, k, seed=810 + n + group)
    _check(W, fmt, group=group)


@pytest.mark.parametrize("nbits", [2, 3, 4, 5, 6, 7])
@pytest.mark.parametrize("dt,group,n,k", [("bf16", 64, 64, 512), ("bf16", 32, 136, 1024), ("f16", 128, 64, 1024),
                                          ("f32", 64, 24, 2048), ("bf16", 64, 10, 128)])
def test_quantize_snr_uintx(nbits, dt, group, n, k):
    """The tiled layout fuses; a shape outside it (10 x 128: not whole 8 x group sets)
    takes the two passes, with the same results."""
    W = workloads.uintx_weight(n, k, seed=820 + n + nbits, outlier_frac=0.01, dtype=_TDT[dt])
    _check(W, "uintx", nbits=nbits, group=group)


def test_quantize_snr_full_34816x5120():
    """The metric weight, MXFP4, GPTQ sym g128 and uintx5 g64: stored tensors and sums as
    the two separate calls."""
    W = workloads.mxfp4_weight()
    Wd = W.to(DEV)
    for fmt, nb, g in (("mxfp4", 4, None), ("gptq_sym", 4, 128), ("uintx", 5, 64)):
        q1 = gwb.quantize(Wd, fmt, nbits=nb, group=g)
        s1 = gwb.snr(Wd, q1).cpu().numpy()
        q2, s2 = gwb.quantize_snr(Wd, fmt, nbits=nb, group=g)
        s2 = s2.cpu().numpy()
        assert torch.equal(q1.codes, q2.codes) and torch.equal(q1.scales, q2.scales), fmt
        assert s2[0] == pytest.approx(s1[0], rel=1e-12) and s2[1] == pytest.approx(s1[1], rel=1e-12), fmt
        del q1, q2
