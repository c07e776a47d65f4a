"""C ABI boundary checks that need no GPU: libgwb.so loads, exports every entry point
include/gwb.h declares, reports the documented sizes, and rejects bad arguments with the
documented codes before anything is enqueued (so no HIP call is reached here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gwb.h")

gwb = pytest.importorskip("group_wise_bit_amd.binding", reason="libgwb.so not built")
lib = gwb.lib


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(gwb_[a-z0-9_]+)\s*\(", txt)))


def test_header_declares_what_binding_exports():
    declared = _declared()
    assert declared, "no declarations found"
    assert set(declared) == set(gwb.EXPORTS)


def test_library_exports_every_declared_symbol():
    for name in _declared():
        assert hasattr(lib, name), name


def _sizes(fmt, N, K, nbits=4, group=None, dt=gwb.BF16):
    sp = gwb.make_spec(fmt, nbits, group, dt)
    s = gwb.Sizes()
    rc = lib.gwb_query_sizes(ctypes.byref(sp), N, K, ctypes.byref(s))
    return rc, s


def test_sizes_match_layouts():
    rc, s = _sizes("mxfp4", 34816, 5120)
    assert rc == 0 and s.codes == 34816 * 2560 and s.scales == 34816 * 160 and s.zeros == 0
    rc, s = _sizes("gptq_sym", 256, 1024, dt=gwb.F32)
    assert rc == 0 and (s.codes, s.scales, s.zeros, s.g_idx) == (128 * 256 * 4, 8 * 256 * 2, 8 * 32 * 4, 1024 * 4)
    rc, s = _sizes("gptq_asym", 4096, 4096)
    assert rc == 0 and (s.codes, s.scales, s.zeros) == (512 * 4096 * 4, 32 * 4096 * 2, 32 * 512 * 4)
    for nbits, want in [(2, 9437184), (3, 14155776), (4, 18874368), (5, 23592960), (6, 28311552), (7, 33030144)]:
        rc, s = _sizes("uintx", 3072, 12288, nbits=nbits)
        assert rc == 0 and s.codes == want and s.scales == 1179648 and s.zeros == 589824
    # ragged uintx: shards padded independently, workspace for the two-pass path
    rc, s = _sizes("uintx", 1, 64, nbits=5)
    assert rc == 0 and s.codes == 32 + 8 and s.workspace >= 64
    # the uintx scale has the weight dtype; groups 32 and 128. N*K % (8 group) == 0 takes
    # the tiled kernels (error partials only), other shapes the two-pass path (a codes
    # workspace of N*K bytes)
    rc, s = _sizes("uintx", 64, 512, nbits=4, group=32, dt=gwb.F32)
    assert rc == 0 and s.scales == 64 * 16 * 4 and s.zeros == 64 * 16 and s.workspace < 64 * 512
    rc, s = _sizes("uintx", 64, 512, nbits=3, group=128, dt=gwb.F16)
    assert rc == 0 and s.scales == 64 * 4 * 2 and s.zeros == 64 * 4 and s.codes == 64 * 512 * 3 // 8
    assert s.workspace < 64 * 512
    rc, s = _sizes("uintx", 3, 256, nbits=3, group=128, dt=gwb.F16)      # 768 % 1024 != 0
    assert rc == 0 and s.workspace >= 3 * 256
    rc, s = _sizes("uintx", 3, 256, nbits=3, group=32, dt=gwb.F16)       # 768 % 256 == 0
    assert rc == 0 and s.workspace < 3 * 256


def test_bits_per_weight_from_sizes():
    # page export_gptq_cpu.py main: 4 + (16 + 4) / group bits per weight
    rc, s = _sizes("gptq_asym", 4096, 4096)
    bpw = 8 * (s.codes + s.scales + s.zeros) / (4096 * 4096)
    assert bpw == 4 + 20 / 128


@pytest.mark.parametrize("fmt,N,K,nbits,group,dt,code", [
    ("mxfp4", 4, 48, 4, 32, gwb.BF16, gwb.E_SHAPE),
    ("mxfp4", 4, 64, 4, 16, gwb.BF16, gwb.E_UNSUPPORTED),
    ("mxfp4", 4, 64, 3, 32, gwb.BF16, gwb.E_ARG),
    ("gptq_sym", 4, 128, 4, 128, gwb.F32, gwb.E_SHAPE),       # N % 8
    ("gptq_sym", 8, 192, 4, 128, gwb.F32, gwb.E_SHAPE),       # K % group
    ("gptq_asym", 8, 128, 4, 256, gwb.BF16, gwb.E_UNSUPPORTED),
    ("gptq_asym", 8, 128, 4, 0, gwb.BF16, gwb.E_ARG),
    ("gptq_asym", 8, 128, 3, 128, gwb.BF16, gwb.E_ARG),
    ("uintx", 8, 128, 8, 64, gwb.BF16, gwb.E_UNSUPPORTED),    # uint8 refused
    ("uintx", 8, 128, 1, 64, gwb.BF16, gwb.E_ARG),
    ("uintx", 8, 100, 4, 64, gwb.BF16, gwb.E_SHAPE),
    ("uintx", 8, 128, 4, 16, gwb.F16, gwb.E_UNSUPPORTED),     # groups 32, 64, 128
    ("uintx", 8, 128, 4, 0, gwb.F32, gwb.E_ARG),
    ("uintx", 8, 96, 4, 64, gwb.F16, gwb.E_SHAPE),
    ("uintx", 8, 128, 4, 64, 3, gwb.E_ARG),                   # unknown dtype
    ("mxfp4", 8, 128, 4, 32, gwb.F16, gwb.E_UNSUPPORTED),     # float16 weights: uintx only
    ("gptq_sym", 8, 128, 4, 128, gwb.F16, gwb.E_UNSUPPORTED),
    ("uintx", -1, 128, 4, 64, gwb.BF16, gwb.E_ARG),
    ("mxfp4", 1 << 21, 1 << 16, 4, 32, gwb.BF16, gwb.E_UNSUPPORTED),   # 2^37 elements: past MXFP4's row bands
    ("gptq_sym", 1 << 16, 1 << 16, 4, 128, gwb.BF16, gwb.E_UNSUPPORTED),   # 2^32: GPTQ indexes below 2^31
    ("uintx", 1 << 16, 1 << 16, 4, 64, gwb.BF16, gwb.E_UNSUPPORTED),
])
def test_query_rejects(fmt, N, K, nbits, group, dt, code):
    rc, _ = _sizes(fmt, N, K, nbits, group, dt)
    assert rc == code
    assert lib.gwb_last_error().decode()


def test_mxfp4_row_bands_past_2_31():
    """MXFP4 shapes of 2^31 elements or more are accepted by the size query, quantize,
    dequantize and SNR (row bands of fewer than 2^31 elements each); sizes are those of
    the whole layout, and the workspace holds every band's partials. The GEMV, GEMM and
    fold keep the 2^31 limit."""
    N, K = 131080, 16384                      # 2^31 + 131072 elements: bands of 131071 and 9 rows
    rc, sz = _sizes("mxfp4", N, K, 4, 32, gwb.BF16)
    assert rc == gwb.OK
    assert sz.codes == N * K // 2 and sz.scales == N * K // 32
    rc1, sz1 = _sizes("mxfp4", 131071, K, 4, 32, gwb.BF16)
    rc2, sz2 = _sizes("mxfp4", 9, K, 4, 32, gwb.BF16)
    assert rc1 == rc2 == gwb.OK and sz.workspace == sz1.workspace + sz2.workspace
    sp, b = gwb.make_spec("mxfp4", 4, 32, gwb.BF16), ctypes.c_size_t()
    assert lib.gwb_gemv_workspace(ctypes.byref(sp), N, K, 1, ctypes.byref(b)) == gwb.E_UNSUPPORTED
    assert lib.gwb_gemm_workspace(ctypes.byref(sp), N, K, 16, ctypes.byref(b)) == gwb.E_UNSUPPORTED


def test_unknown_format_and_dtype():
    s = gwb.Sizes()
    assert lib.gwb_query_sizes(ctypes.byref(gwb.QSpec(10, 4, 32, 1)), 8, 64, ctypes.byref(s)) == gwb.E_ARG
    assert lib.gwb_query_sizes(ctypes.byref(gwb.QSpec(0, 4, 32, 1)), 8, 64, ctypes.byref(s)) == gwb.E_ARG
    assert lib.gwb_query_sizes(ctypes.byref(gwb.QSpec(3, 4, 32, 7)), 8, 64, ctypes.byref(s)) == gwb.E_ARG
    assert lib.gwb_query_sizes(None, 8, 64, ctypes.byref(s)) == gwb.E_ARG


def test_quantize_validates_before_launch():
    sp = gwb.make_spec("mxfp4", 4, 32, gwb.BF16)
    fake = 1 << 20          # never dereferenced: every call below fails validation first
    qt = gwb.QTensors(fake, fake, None, None)
    assert lib.gwb_quantize(ctypes.byref(sp), None, 8, 64, 64, ctypes.byref(qt), None, 0, None) == gwb.E_ARG
    assert lib.gwb_quantize(ctypes.byref(sp), fake, 8, 64, 32, ctypes.byref(qt), None, 0, None) == gwb.E_ARG
    assert lib.gwb_quantize(ctypes.byref(sp), fake + 2, 8, 64, 64, ctypes.byref(qt), None, 0, None) == gwb.E_UNSUPPORTED
    assert lib.gwb_quantize(ctypes.byref(sp), fake, 8, 64, 68, ctypes.byref(qt), None, 0, None) == gwb.E_UNSUPPORTED
    bad = gwb.QTensors(None, fake, None, None)
    assert lib.gwb_quantize(ctypes.byref(sp), fake, 8, 64, 64, ctypes.byref(bad), None, 0, None) == gwb.E_ARG
    # uintx two-pass path needs its workspace
    su = gwb.make_spec("uintx", 3, 64, gwb.BF16)
    qu = gwb.QTensors(fake, fake, fake, None)
    assert lib.gwb_quantize(ctypes.byref(su), fake, 1, 64, 64, ctypes.byref(qu), None, 0, None) == gwb.E_SIZE
    # GPTQ needs zeros
    sg = gwb.make_spec("gptq_sym", 4, 128, gwb.F32)
    assert lib.gwb_quantize(ctypes.byref(sg), fake, 8, 128, 128, ctypes.byref(qt), None, 0, None) == gwb.E_ARG
    # empty shapes are valid and enqueue nothing
    assert lib.gwb_quantize(ctypes.byref(sp), fake, 0, 64, 64, ctypes.byref(qt), None, 0, None) == gwb.OK
    assert lib.gwb_quantize(ctypes.byref(sp), fake, 8, 0, 0, ctypes.byref(qt), None, 0, None) == gwb.OK


def test_dequantize_snr_awq_validate():
    fake = 1 << 20
    sp = gwb.make_spec("mxfp4", 4, 32, gwb.BF16)
    qt = gwb.QTensors(fake, fake, None, None)
    assert lib.gwb_dequantize(ctypes.byref(sp), ctypes.byref(qt), 8, 64, fake, 5, 64, None, 0, None) == gwb.E_ARG
    assert lib.gwb_dequantize(ctypes.byref(sp), ctypes.byref(qt), 8, 64, fake, gwb.BF16, 32, None, 0, None) == gwb.E_ARG
    assert lib.gwb_dequantize(ctypes.byref(sp), ctypes.byref(qt), 8, 64, None, gwb.BF16, 64, None, 0, None) == gwb.E_ARG
    assert lib.gwb_dequantize(ctypes.byref(sp), ctypes.byref(qt), 8, 64, fake, gwb.F16, 64, None, 0, None) \
        == gwb.E_UNSUPPORTED                                   # float16 output: uintx only
    # uintx values are of the weight dtype: float32 or that dtype out, nothing else
    qu = gwb.QTensors(fake, fake, fake, None)
    for wdt, odt in [(gwb.F16, gwb.BF16), (gwb.F32, gwb.BF16), (gwb.F32, gwb.F16), (gwb.BF16, gwb.F16)]:
        su = gwb.make_spec("uintx", 4, 64, wdt)
        assert lib.gwb_dequantize(ctypes.byref(su), ctypes.byref(qu), 8, 64, fake, odt, 64, None, 0, None) \
            == gwb.E_UNSUPPORTED, (wdt, odt)
    assert lib.gwb_snr(ctypes.byref(sp), fake, 8, 64, 64, ctypes.byref(qt), fake, None, 0, None) == gwb.E_SIZE
    assert lib.gwb_snr(ctypes.byref(sp), fake, 0, 64, 64, ctypes.byref(qt), fake, fake, 1 << 20, None) == gwb.E_SHAPE
    al = (ctypes.c_double * 11)(*[i / 10 for i in range(11)])
    args = dict(W=fake, dt=gwb.BF16, N=64, K=64, ldw=64, a=fake, al=al, na=11, mr=2048, s=fake, e=fake, b=fake)
    def awq(**kw):
        a = dict(args, **kw)
        return lib.gwb_awq_search_mxfp4(a["W"], a["dt"], a["N"], a["K"], a["ldw"], a["a"], a["al"], a["na"], a["mr"],
                                        a["s"], a["e"], a["b"], None, 0, None)
    assert awq() == gwb.E_SIZE
    assert awq(K=48) == gwb.E_SHAPE
    assert awq(na=17) == gwb.E_ARG
    assert awq(na=0) == gwb.E_ARG
    assert awq(mr=0) == gwb.E_ARG
    assert awq(a=None) == gwb.E_ARG
    b = ctypes.c_size_t()
    assert lib.gwb_awq_workspace(34816, 5120, 11, 2048, ctypes.byref(b)) == 0 and b.value > 0
    assert lib.gwb_stream_bench(0, 64, fake, fake, 24, None) == gwb.E_UNSUPPORTED
    assert lib.gwb_stream_bench(8, 64, fake, fake, 1 << 20, None) == gwb.E_ARG
    assert lib.gwb_stream_bench(0, 0, fake, fake, 1 << 20, None) == gwb.E_ARG
    assert lib.gwb_stream_bench(1, 2048, fake, fake, 1 << 20, None) == gwb.E_SIZE


def test_error_message_is_thread_local_and_cleared():
    _sizes("uintx", 8, 128, nbits=8)
    assert "uint8" in lib.gwb_last_error().decode()
    rc, _ = _sizes("mxfp4", 8, 64)
    assert rc == 0 and lib.gwb_last_error().decode() == ""


def test_awq_scales_host_matches_oracle_table():
    """Host scaling table (no device memory touched) against the oracle's: float64
    steps rounded once to float32, so at most one float32 ulp apart (summation order)."""
    import numpy as np
    import torch
    import oracle.awq as oawq
    from group_wise_bit_amd import workloads
    for K, seed in ((5120, 5), (96, 71), (1, 72)):
        a = workloads.awq_activation_stat(K, seed=seed)
        got = gwb.awq_scales_host(a).numpy()
        want = oawq.scale_table(a.numpy())
        ulps = np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
        assert ulps.max() <= 1, (K, ulps.max())
        assert np.all(got[0] == 1.0)                       # alpha = 0: s is exactly 1
    flat = gwb.awq_scales_host(torch.full((64,), 0.3))    # constant a: every alpha gives s = 1
    assert torch.all(flat == 1.0)


def test_awq_scales_host_rejects():
    out = (ctypes.c_float * 64)()
    a = (ctypes.c_float * 8)(*([1.0] * 8))
    al = (ctypes.c_double * 17)(*([0.5] * 17))
    f = lib.gwb_awq_scales_host
    assert f(None, 8, ctypes.cast(al, ctypes.c_void_p), 1, ctypes.cast(out, ctypes.c_void_p)) == gwb.E_ARG
    assert f(ctypes.cast(a, ctypes.c_void_p), 0, ctypes.cast(al, ctypes.c_void_p), 1,
             ctypes.cast(out, ctypes.c_void_p)) == gwb.E_ARG
    assert f(ctypes.cast(a, ctypes.c_void_p), 8, ctypes.cast(al, ctypes.c_void_p), 17,
             ctypes.cast(out, ctypes.c_void_p)) == gwb.E_ARG
    assert f(ctypes.cast(a, ctypes.c_void_p), 8, ctypes.cast(al, ctypes.c_void_p), 0,
             ctypes.cast(out, ctypes.c_void_p)) == gwb.E_ARG
    assert b"n_alpha" in lib.gwb_last_error()


def test_fold_validates_before_launch():
    """Every invalid call returns its code before anything is enqueued (dummy device
    addresses are never touched)."""
    P = ctypes.c_void_p
    fake = P(1 << 20)                                  # 16-byte aligned, never dereferenced
    mx = gwb.QTensors(fake.value, fake.value, None, None)
    f = gwb.Fold(fake.value, fake.value, 1, 2)
    call = lib.gwb_fold_mxfp4
    def go(dt=gwb.BF16, N=8, K=64, ldw=64, fold=f, out=fake, ldo=64, q=mx):
        return call(fake, dt, N, K, ldw, None if fold is None else ctypes.byref(fold), out, ldo,
                    None if q is None else ctypes.byref(q), None)
    assert go(dt=gwb.F32) == gwb.E_UNSUPPORTED
    assert go(out=None, q=None) == gwb.E_ARG
    assert go(K=40) == gwb.E_SHAPE                      # MXFP4 output needs K % 32 == 0
    assert go(K=36, ldw=40, q=None, ldo=40) == gwb.E_SHAPE
    assert go(fold=gwb.Fold(fake.value, fake.value, 3, 0)) == gwb.E_ARG
    assert go(fold=gwb.Fold(None, fake.value, 1, 0)) == gwb.E_ARG
    assert go(fold=gwb.Fold(fake.value, None, 0, 2)) == gwb.E_ARG
    assert go(ldw=60) == gwb.E_ARG
    assert go(ldw=68) == gwb.E_UNSUPPORTED
    assert go(ldo=60) == gwb.E_UNSUPPORTED
    assert go(N=0) == gwb.OK and go(K=0) == gwb.OK      # empty: nothing to do
    assert go(N=1 << 20, K=1 << 12, ldw=1 << 12, ldo=1 << 12) == gwb.E_UNSUPPORTED


def test_quantize_snr_validation():
    P = ctypes.c_void_p
    fake = 1 << 20
    qt = gwb.QTensors(fake, fake, fake, None)
    sp = gwb.make_spec("mxfp4", 4, 32)
    def go(spec=sp, N=64, K=256, W=fake, d=fake, ws=fake, wsb=1 << 20):
        return lib.gwb_quantize_snr(ctypes.byref(spec), P(W), N, K, K, ctypes.byref(qt), P(d), P(ws), wsb, None)
    assert go(d=None) == gwb.E_ARG
    assert go(N=0) == gwb.E_SHAPE and go(K=0) == gwb.E_SHAPE
    assert go(wsb=16) == gwb.E_SIZE
    assert go(ws=fake + 8) == gwb.E_UNSUPPORTED
    assert go(spec=gwb.make_spec("gptq_sym_act", 4, 128)) == gwb.E_ARG
    # shapes the fused kernels do not cover run quantize and SNR as two calls; the
    # workspace of both is checked before the first launch (fake pointers: a launch here
    # would fail, a short workspace must be refused first)
    big = gwb.make_spec("gptq_sym", 4, 128)
    assert go(spec=big, N=131072, K=4096, wsb=64) == gwb.E_SIZE
    ux = gwb.make_spec("uintx", 5, 64)
    assert go(spec=ux, N=10, K=128, wsb=256) == gwb.E_SIZE       # two-pass codes need N*K bytes


def test_gemv_sizes_and_validation():
    P = ctypes.c_void_p
    fake = 1 << 20
    qt = gwb.QTensors(fake, fake, fake, None)
    def ws(fmt, N, K, B, group=None, dt=gwb.BF16, nbits=4):
        sp, b = gwb.make_spec(fmt, nbits, group, dt), ctypes.c_size_t()
        rc = lib.gwb_gemv_workspace(ctypes.byref(sp), N, K, B, ctypes.byref(b))
        return rc, b.value
    assert ws("gptq_sym", 131072, 2048, 1) == (gwb.OK, 0)                  # 512 column tiles: one split
    assert ws("gptq_sym", 65536, 2048, 1) == (gwb.OK, 4 * 65536 * 4)        # 256 tiles: four K splits (~1024 blocks)
    assert ws("gptq_sym", 34816, 5120, 1) == (gwb.OK, 5 * 34816 * 4)        # 136 tiles: 1024 k per split, 5 splits
    # B >= 2 GPTQ may take the GEMM tiles: the larger of the two needs.
    # GPTQ asym g64 256 x 640, B = 3: GEMV 2 splits x 3 x 256 floats; tiles: the group
    # sums (10 groups x 128 padded rows floats) + 2 K splits x 3 x 256 floats
    assert ws("gptq_asym", 256, 640, 3, 64) == (gwb.OK, 10 * 128 * 4 + 2 * 3 * 256 * 4)
    assert ws("gptq_sym", 131072, 2048, 2) == (gwb.OK, 16 * 128 * 4)            # 512 tiles: no split
    assert ws("gptq_asym", 256, 576, 3, 64) == (gwb.OK, 2 * 3 * 256 * 4)      # K % 128 != 0: GEMV only
    assert ws("mxfp4", 4096, 2048, 4) == (gwb.OK, 0)                          # the GEMV: no workspace
    # 5 to 8 rows: the matrix-core GEMV, K splits of at most 2048 k (8 rows) or 3072 (5)
    assert ws("mxfp4", 4096, 2048, 8) == (gwb.OK, 0)
    assert ws("mxfp4", 34816, 5120, 8) == (gwb.OK, 3 * 8 * 34816 * 4)
    assert ws("mxfp4", 34816, 5120, 5) == (gwb.OK, 2 * 5 * 34816 * 4)
    assert ws("gptq_sym", 256, 512, 0)[0] == gwb.E_ARG
    assert ws("gptq_sym", 256, 512, 9)[0] == gwb.E_ARG
    sp_u = gwb.make_spec("uintx", 4, 64)
    assert lib.gwb_gemv_workspace(ctypes.byref(sp_u), 64, 128, 1, ctypes.byref(ctypes.c_size_t())) == gwb.E_UNSUPPORTED
    assert lib.gwb_gemv_workspace(ctypes.byref(sp_u), 12, 512, 1, ctypes.byref(ctypes.c_size_t())) == gwb.E_UNSUPPORTED
    # bf16 uintx2/4 from 2 rows (3, 5, 6 bits from 3, 7 bits from 5): the matrix-core decode
    # kernel, 24 blocks of 16 x 8 rows -> K splits toward 1024 blocks, at least 2 batches of 256 k
    assert ws("uintx", 3072, 12288, 2) == (gwb.OK, 24 * 2 * 3072 * 4)
    # the GEMV kernels (fp16 weights): 2048 columns per wavefront up to 4 rows, 1024 or 512 beyond
    assert ws("uintx", 3072, 12288, 4, 64, gwb.F16) == (gwb.OK, 6 * 4 * 3072 * 4)
    assert ws("uintx", 3072, 12288, 8, 64, gwb.F16) == (gwb.OK, 12 * 8 * 3072 * 4)
    assert ws("uintx", 3072, 11776, 8, 64, gwb.F16) == (gwb.OK, 23 * 8 * 3072 * 4)   # K % 1024 != 0
    assert ws("uintx", 3072, 12288, 8) == (gwb.OK, 24 * 8 * 3072 * 4)             # bf16: the decode kernel
    assert ws("uintx", 3072, 12288, 8, 64, gwb.BF16, 7) == (gwb.OK, 24 * 8 * 3072 * 4)
    assert ws("uintx", 3072, 12288, 4, 64, gwb.BF16, 7) == (gwb.OK, 6 * 4 * 3072 * 4)    # 7 bits, 4 rows: the GEMV
    # bf16 uintx4 on the 131072 x 2048 head: 1024 decode blocks, no split; the size still
    # covers the GEMV's (2 splits), which takes the call when the packed codes are not
    # 16-byte aligned
    assert ws("uintx", 131072, 2048, 8) == (gwb.OK, 2 * 8 * 131072 * 4)
    assert ws("uintx", 131072, 4096, 8) == (gwb.OK, 4 * 8 * 131072 * 4)           # GEMV: 4 splits
    assert ws("uintx", 131072, 2048, 4) == (gwb.OK, 0)
    assert ws("uintx", 131072, 2048, 8, 64, gwb.BF16, 7) == (gwb.OK, 2 * 8 * 131072 * 4)
    assert ws("uintx", 64, 1536, 1) == (gwb.OK, 3 * 64 * 4)                      # 512-column splits
    assert ws("uintx", 131072, 2048, 1) == (gwb.OK, 0)                           # one split: y directly
    for g, dt in [(32, gwb.BF16), (64, gwb.F16), (128, gwb.F32)]:                # every dtype and group
        su, b = gwb.make_spec("uintx", 4, g, dt), ctypes.c_size_t()
        assert lib.gwb_gemv_workspace(ctypes.byref(su), 64, 1536, 1, ctypes.byref(b)) == gwb.OK
        assert b.value == 3 * 64 * 4
    sp = gwb.make_spec("gptq_sym", 4, 128)
    def go(x=fake, B=1, ldx=1024, y=fake, ydt=gwb.F32, ldy=256, w=0, wsb=0):
        return lib.gwb_gemv(ctypes.byref(sp), ctypes.byref(qt), 256, 1024, P(x), B, ldx, P(y), ydt, ldy, P(w), wsb,
                            None)
    assert go(ydt=7) == gwb.E_ARG
    assert go(x=None) == gwb.E_ARG
    assert go(ldx=1000) == gwb.E_ARG
    assert go(ldx=1028) == gwb.E_UNSUPPORTED
    assert go(x=fake + 4) == gwb.E_UNSUPPORTED
    assert go() == gwb.E_SIZE                                                 # K-split partials needed
    assert go(w=fake + 8, wsb=1 << 20) == gwb.E_UNSUPPORTED


def test_gemm_sizes_and_validation():
    P = ctypes.c_void_p
    fake = 1 << 20
    qt = gwb.QTensors(fake, fake, fake, None)
    def ws(fmt, N, K, M, group=None, dt=gwb.BF16):
        sp, b = gwb.make_spec(fmt, 4, group, dt), ctypes.c_size_t()
        rc = lib.gwb_gemm_workspace(ctypes.byref(sp), N, K, M, ctypes.byref(b))
        return rc, b.value
    assert ws("gptq_sym", 34816, 5120, 2048) == (gwb.OK, 40 * 2048 * 4)       # group sums, rows padded to 128
    assert ws("gptq_asym", 4096, 4096, 100, 32) == (gwb.OK, 128 * 128 * 4)
    assert ws("mxfp4", 34816, 5120, 2048) == (gwb.OK, 0)
    assert ws("mxfp4_page_ties", 256, 128, 1) == (gwb.OK, 0)
    assert ws("gptq_sym", 256, 1024, 0) == (gwb.OK, 0)
    assert ws("mxfp4", 264, 2048, 16) == (gwb.OK, 4 * 16 * 264 * 4)            # small M: 4 K splits
    assert ws("gptq_sym", 264, 2048, 16, 128) == (gwb.OK, 16 * 128 * 4 + 4 * 16 * 264 * 4)
    assert ws("mxfp4", 34816, 640, 64) == (gwb.OK, 2 * 64 * 34816 * 4)         # 5 stages: 2 splits
    assert ws("mxfp4", 131072, 2048, 64) == (gwb.OK, 0)                        # 512 tiles: no split
    assert ws("gptq_sym", 256, 576, 16, 64)[0] == gwb.E_UNSUPPORTED           # K % 128
    assert ws("mxfp4", 100, 1024, 16)[0] == gwb.E_UNSUPPORTED                 # N % 8
    # uintx: bf16 weights, N % 8 == 0, K % 512 == 0; 16-row tiles of 64 x 8 weight rows
    assert ws("uintx", 256, 1024, 16, 64) == (gwb.OK, 4 * 16 * 256 * 4)       # 1 block: 4 = 8 stages / 2
    assert ws("uintx", 3072, 12288, 8, 64) == (gwb.OK, 32 * 8 * 3072 * 4)     # 6 blocks: 32 splits
    assert ws("uintx", 131072, 2048, 8, 64) == (gwb.OK, 2 * 8 * 131072 * 4)   # 256 blocks: 2 splits
    assert ws("uintx", 131072, 2048, 64, 64) == (gwb.OK, 0)                   # 1024 blocks
    assert ws("uintx", 256, 1152, 16, 64)[0] == gwb.E_UNSUPPORTED             # K % 512
    assert ws("uintx", 256, 1024, 16, 64, gwb.F16)[0] == gwb.E_UNSUPPORTED    # fp16 weights
    assert ws("gptq_sym_act", 256, 1024, 16, 128)[0] == gwb.E_UNSUPPORTED
    assert ws("gptq_sym", 256, 1024, -1)[0] == gwb.E_ARG
    assert ws("gptq_sym", 256, 1024, (1 << 24) + 1)[0] == gwb.E_ARG
    assert ws("gptq_sym", 256, 1 << 20, 1 << 11)[0] == gwb.E_UNSUPPORTED       # M*K = 2^31
    sp = gwb.make_spec("gptq_sym", 4, 128)
    def go(x=fake, M=16, ldx=1024, y=fake, ydt=gwb.F32, ldy=256, w=fake, wsb=1 << 20, q=qt):
        return lib.gwb_gemm(ctypes.byref(sp), ctypes.byref(q), 256, 1024, P(x), M, ldx, P(y), ydt, ldy, P(w), wsb,
                            None)
    assert go(ydt=7) == gwb.E_ARG
    assert go(x=None) == gwb.E_ARG
    assert go(ldx=1000) == gwb.E_ARG
    assert go(ldy=200) == gwb.E_ARG
    assert go(ldx=1028) == gwb.E_UNSUPPORTED
    assert go(x=fake + 4) == gwb.E_UNSUPPORTED
    assert go(y=fake + 8) == gwb.E_UNSUPPORTED
    assert go(ldy=260) == gwb.E_UNSUPPORTED
    assert go(q=gwb.QTensors(fake + 4, fake, fake, None)) == gwb.E_UNSUPPORTED
    assert go(w=None, wsb=0) == gwb.E_SIZE                                      # group sums needed
    assert go(wsb=100) == gwb.E_SIZE
    assert go(w=fake + 8) == gwb.E_UNSUPPORTED
    assert go(M=0, x=None, y=None) == gwb.OK                                    # empty: nothing to do


def test_page_ties_format_shares_mxfp4_sizes():
    for N, K in ((34816, 5120), (3, 96)):
        a = gwb.query_sizes("mxfp4", N, K, 4, 32)
        b = gwb.query_sizes("mxfp4_page_ties", N, K, 4, 32)
        assert a == b
    sp = gwb.make_spec("mxfp4_page_ties", 4, 32)
    assert lib.gwb_query_sizes(ctypes.byref(sp), 8, 48, ctypes.byref(gwb.Sizes())) == gwb.E_SHAPE


def test_act_order_gptq_validates():
    fake = 1 << 20
    P = ctypes.c_void_p
    rc, s = _sizes("gptq_sym_act", 256, 1024, group=32)
    rc2, s2 = _sizes("gptq_sym", 256, 1024, group=32)
    assert rc == 0 and (s.codes, s.scales, s.zeros, s.g_idx) == (s2.codes, s2.scales, s2.zeros, s2.g_idx)
    assert s.workspace >= 256 * 32 * 5                             # float32 scale + zero point per (row, group)
    assert _sizes("gptq_asym_act", 8, 32 * 257, group=32)[0] == gwb.E_UNSUPPORTED   # > 256 groups per row
    assert _sizes("gptq_asym_act", 8, 32 * 256, group=32)[0] == gwb.OK
    assert _sizes("gptq_asym_act", 8, 32768, group=128)[0] == gwb.OK                 # a 64 KB bf16 row
    assert _sizes("gptq_asym_act", 8, 32768, group=128, dt=gwb.F32)[0] == gwb.E_UNSUPPORTED
    sp = gwb.make_spec("gptq_asym_act", 4, 128, gwb.BF16)
    qt = gwb.QTensors(fake, fake, fake, fake)
    qn = gwb.QTensors(fake, fake, fake, None)
    # plain quantize refuses the act-order formats; the act-order entry refuses the others
    assert lib.gwb_quantize(ctypes.byref(sp), fake, 8, 256, 256, ctypes.byref(qt), fake, 1 << 30, None) == gwb.E_ARG
    def act(spec=sp, perm=fake, q=qt, ws=fake, wsb=1 << 30):
        return lib.gwb_quantize_act_order(ctypes.byref(spec), P(fake), 8, 256, 256, P(perm), ctypes.byref(q), P(ws),
                                          wsb, None)
    assert act(spec=gwb.make_spec("gptq_asym", 4, 128, gwb.BF16)) == gwb.E_ARG
    assert act(perm=None) == gwb.E_ARG
    assert act(q=qn) == gwb.E_ARG                                   # g_idx is an output here
    assert act(wsb=100) == gwb.E_SIZE
    assert act(ws=fake + 8) == gwb.E_UNSUPPORTED
    assert act(perm=fake + 4) == gwb.E_UNSUPPORTED
    # dequantization and SNR need g_idx; the GEMV takes act-order weights
    assert lib.gwb_dequantize(ctypes.byref(sp), ctypes.byref(qn), 8, 256, P(fake), gwb.F32, 256, None, 0, None) \
        == gwb.E_ARG
    assert lib.gwb_snr(ctypes.byref(sp), P(fake), 8, 256, 256, ctypes.byref(qn), P(fake), P(fake), 1 << 20, None) \
        == gwb.E_ARG
    b = ctypes.c_size_t()
    assert lib.gwb_gemv_workspace(ctypes.byref(sp), 8, 256, 1, ctypes.byref(b)) == gwb.OK and b.value == 0
    assert lib.gwb_gemv_workspace(ctypes.byref(sp), 64, 2048, 2, ctypes.byref(b)) == gwb.OK
    assert b.value == 4 * 2 * 64 * 4                                # one column tile: a split per 512 k


def test_group_order_validates():
    """gwb_gptq_group_order takes act-order tensors and validates before enqueueing; the
    group-ordered formats have GPTQ's sizes, are refused by every entry point but
    gwb_gemv, and need their permutation there."""
    fake = 1 << 20
    P = ctypes.c_void_p
    rc, s = _sizes("gptq_sym_grouped", 256, 1024, group=32)
    rc2, s2 = _sizes("gptq_sym", 256, 1024, group=32)
    assert rc == 0 and (s.codes, s.scales, s.zeros, s.g_idx, s.workspace) == (s2.codes, s2.scales, s2.zeros, s2.g_idx, 0)
    act = gwb.make_spec("gptq_sym_act", 4, 128, gwb.BF16)
    qt = gwb.QTensors(fake, fake, fake, fake)
    def go(spec=act, q=qt, out=fake + 4096, perm=fake + 8192, status=fake + 16384, N=64, K=256):
        return lib.gwb_gptq_group_order(ctypes.byref(spec), None if q is None else ctypes.byref(q), N, K, P(out),
                                        P(perm), P(status), None)
    assert go(spec=gwb.make_spec("gptq_sym", 4, 128, gwb.BF16)) == gwb.E_ARG
    assert go(q=None) == gwb.E_ARG
    assert go(q=gwb.QTensors(fake, fake, fake, None)) == gwb.E_ARG      # g_idx is the input
    assert go(out=None) == gwb.E_ARG and go(perm=None) == gwb.E_ARG and go(status=None) == gwb.E_ARG
    assert go(out=fake) == gwb.E_ARG                                    # no in-place rearrangement
    assert go(out=fake + 4100) == gwb.E_UNSUPPORTED
    assert go(K=200) == gwb.E_SHAPE
    assert go(N=0) == gwb.OK and go(K=0) == gwb.OK                      # empty: nothing enqueued
    grp = gwb.make_spec("gptq_asym_grouped", 4, 128, gwb.BF16)
    qn = gwb.QTensors(fake, fake, fake, None)
    assert lib.gwb_quantize(ctypes.byref(grp), fake, 8, 256, 256, ctypes.byref(qt), fake, 1 << 30, None) \
        == gwb.E_UNSUPPORTED
    assert lib.gwb_dequantize(ctypes.byref(grp), ctypes.byref(qt), 8, 256, P(fake), gwb.F32, 256, None, 0, None) \
        == gwb.E_UNSUPPORTED
    assert lib.gwb_snr(ctypes.byref(grp), P(fake), 8, 256, 256, ctypes.byref(qt), P(fake), P(fake), 1 << 20,
                       None) == gwb.E_UNSUPPORTED
    assert lib.gwb_quantize_snr(ctypes.byref(grp), P(fake), 8, 256, 256, ctypes.byref(qt), P(fake), P(fake),
                                1 << 20, None) == gwb.E_UNSUPPORTED
    b = ctypes.c_size_t()
    # the GEMV: gathered activations (256-byte aligned) before index-order GPTQ's own needs
    assert lib.gwb_gemv_workspace(ctypes.byref(grp), 131072, 2048, 1, ctypes.byref(b)) == gwb.OK
    assert b.value == 2048 * 2
    assert lib.gwb_gemv_workspace(ctypes.byref(grp), 64, 2048, 3, ctypes.byref(b)) == gwb.OK
    twin = ctypes.c_size_t()
    assert lib.gwb_gemv_workspace(ctypes.byref(gwb.make_spec("gptq_asym", 4, 128, gwb.BF16)), 64, 2048, 3,
                                  ctypes.byref(twin)) == gwb.OK
    assert b.value == (3 * 2048 * 2 + 255) // 256 * 256 + twin.value
    y = P(fake + (1 << 16))
    assert lib.gwb_gemv(ctypes.byref(grp), ctypes.byref(qn), 64, 2048, P(fake), 1, 2048, y, gwb.F32, 64, P(fake),
                        1 << 20, None) == gwb.E_ARG                     # the permutation is required


def test_static_quantize_snr_rejects_beyond_its_scratch():
    """gwb_quantize_snr_static validates before touching the device: a shape whose
    partials exceed the static array is GWB_E_SIZE, a bad spec keeps its own code."""
    P = ctypes.c_void_p
    fake = 1 << 20
    qt = gwb.QTensors(fake, fake, fake, None)
    ux = gwb.make_spec("uintx", 4, 64)
    # 16384 x 17408 bf16: 17408 tiles of 16384 weights, 16 bytes of partials each > 256 KiB
    assert lib.gwb_quantize_snr_static(ctypes.byref(ux), P(fake), 16384, 17408, 17408, ctypes.byref(qt), P(fake),
                                       None) == gwb.E_SIZE
    assert "static" in lib.gwb_last_error().decode()
    bad = gwb.make_spec("uintx", 8, 64)
    assert lib.gwb_quantize_snr_static(ctypes.byref(bad), P(fake), 64, 512, 512, ctypes.byref(qt), P(fake),
                                       None) == gwb.E_UNSUPPORTED
