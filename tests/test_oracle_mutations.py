"""Planted mistakes in the oracle (CPU only, via monkeypatch) must each fail a pin.
Shows the pins are sharp enough to catch a wrong tie rule, exponent offset, nibble or
shard order, a dropped bfloat16 rounding, a wrong weighting and a wrong sign."""
import numpy as np
import pytest

import oracle.awq as awq
import oracle.gptq as gq
import oracle.mxfp4 as mx
import oracle.snr as snr
import oracle.uintx as ux
import test_oracle_gptq as tg
import test_oracle_mxfp4 as tm
import test_oracle_snr_awq as ts
import test_oracle_uintx as tu


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_mxfp4_page_literal_ties_caught(monkeypatch):
    orig = mx.nearest_index
    monkeypatch.setattr(mx, "nearest_index", lambda m, ties="even": orig(m, "page_literal"))
    _fails(tm.test_ties_go_to_even_code)


def test_mxfp4_exponent_offset_caught(monkeypatch):
    orig = mx.block_exponent
    monkeypatch.setattr(mx, "block_exponent", lambda a: np.clip(orig(a) + 1, -127, 127))
    _fails(tm.test_worked_example_block)
    _fails(tm.test_invariants_block_max_lands_at_top)


def test_mxfp4_nibble_order_caught(monkeypatch):
    orig = mx.unpack_codes
    def swapped(p):
        c = orig(p)
        out = c.copy()
        out[:, 0::2], out[:, 1::2] = c[:, 1::2], c[:, 0::2]
        return out
    monkeypatch.setattr(mx, "unpack_codes", swapped)
    _fails(tm.test_bruteforce_exact_random_and_adversarial, __import__("torch").float32)


def test_gptq_pack_order_caught(monkeypatch):
    orig = gq.pack_int32
    def high_first(c, dim):
        c = np.asarray(c)
        c = c[::-1] if dim == 0 else c[:, ::-1]
        return orig(np.ascontiguousarray(c), dim)
    monkeypatch.setattr(gq, "pack_int32", high_first)
    _fails(tg.test_pack_int32_examples)


def test_gptq_sym_offset_caught(monkeypatch):
    orig = gq.quantize_sym
    def off7(w, group=128):
        q = orig(w, group)
        q["codes"] = np.clip(q["codes"].astype(int) - 1, 0, 15).astype(np.uint8)
        q["qweight"] = gq.pack_int32(q["codes"], 0)
        return q
    monkeypatch.setattr(gq, "quantize_sym", off7)
    _fails(tg.test_worked_example_sym)
    _fails(tg.test_sym_bruteforce_exact, 128)


def test_gptq_asym_zero_minus_one_caught(monkeypatch):
    orig = gq.quantize_asym
    def zm1(w, group=128):
        q = orig(w, group)
        q["qzeros"] = gq.pack_int32(np.clip(q["zp"].astype(int) - 1, 0, 15).astype(np.uint8), 1)
        return q
    monkeypatch.setattr(gq, "quantize_asym", zm1)
    _fails(tg.test_worked_example_asym)


def test_uintx_shard_order_caught(monkeypatch):
    monkeypatch.setattr(ux, "SHARD_WIDTHS", (1, 2, 4, 8))
    _fails(tu.test_pack_worked_examples)


def test_uintx_dropped_bf16_rounding_caught(monkeypatch):
    monkeypatch.setattr(ux, "bf", lambda x: np.asarray(x, np.float32))
    _fails(tu.test_quantize_bruteforce_exact, 5)


def test_gptq_g_idx_ignored_caught(monkeypatch):
    orig = gq.dequantize
    monkeypatch.setattr(gq, "dequantize", lambda qw, s, qz, group, sym, g_idx=None: orig(qw, s, qz, group, sym))
    _fails(tg.test_dequant_g_idx_exact, False)


def test_gptq_act_order_groups_in_index_order_caught(monkeypatch):
    orig = gq.quantize_act_order
    monkeypatch.setattr(gq, "quantize_act_order", lambda w, group, sym, perm: orig(w, group, sym, np.sort(perm)))
    _fails(tg.test_act_order_bruteforce_exact, True)


def test_uintx_float16_rounded_as_bf16_caught(monkeypatch):
    monkeypatch.setattr(ux, "f16", ux.bf)
    _fails(tu.test_quantize_bruteforce_exact_other_dtypes, "f16", 4, 64)


def test_uintx_float32_rounded_as_bf16_caught(monkeypatch):
    orig = ux.rounder
    monkeypatch.setattr(ux, "rounder", lambda d: orig("bf16") if d == "f32" else orig(d))
    _fails(tu.test_quantize_bruteforce_exact_other_dtypes, "f32", 2, 32)


def test_awq_wrong_weighting_caught(monkeypatch):
    orig = awq.clamp_stat
    monkeypatch.setattr(awq, "clamp_stat", lambda a: (orig(a) / orig(a).mean()).astype(np.float32))
    _fails(ts.test_weighted_error_bruteforce_exact)


def test_snr_wrong_sign_caught(monkeypatch):
    def plus(w, d):
        w = np.asarray(w, np.float32); d = np.asarray(d, np.float32)
        e = (w + d).astype(np.float64)
        return float(np.sum(w.astype(np.float64) ** 2)), float(np.sum(e * e))
    monkeypatch.setattr(snr, "sums", plus)
    _fails(ts.test_snr_closed_form_relative_perturbation)


def test_fold_dropped_rounding_caught(monkeypatch):
    import oracle.fold as fd
    import test_oracle_fold as tf
    monkeypatch.setattr(fd, "_apply", lambda x, v, op: x if op == "none" or v is None else (x * v if op == "mul" else x / v))
    _fails(tf.test_each_step_is_one_rounding_of_the_exact_result)


def test_fold_transposed_row_vector_caught(monkeypatch):
    import oracle.fold as fd
    import test_oracle_fold as tf
    orig = fd.fold
    def swapped(w, col=None, col_op="none", row=None, row_op="none"):
        x = orig(w, col, col_op)
        if row_op == "none":
            return x
        return fd._apply(x, np.resize(np.asarray(row, np.float32), x.shape[1])[None, :], row_op)
    monkeypatch.setattr(fd, "fold", swapped)
    _fails(tf.test_orientation_and_order)


def test_gemv_transposed_weight_caught(monkeypatch):
    import oracle.gemv as og
    import test_oracle_gemv as tgv
    monkeypatch.setattr(og, "gemv", lambda deq, x: np.asarray(x, np.float64).reshape(-1, np.shape(deq)[0])
                        @ np.asarray(deq, np.float64) if np.shape(x)[-1] == np.shape(deq)[0]
                        else np.zeros((np.atleast_2d(x).shape[0], np.shape(deq)[0])))
    _fails(tgv.test_orientation_and_linearity)


def test_gptq_page_snr_with_fp16_scale_caught(monkeypatch):
    """The page's in-function SNR formed with the stored fp16 scale instead of the
    float32 one must fail the closed-form pin."""
    for name, sym in (("quantize_sym", True), ("quantize_asym", False)):
        orig = getattr(gq, name)
        def fp16_snr(w, group=128, _orig=orig, _sym=sym):
            q = _orig(w, group)
            d = gq.dequantize(q["qweight"], q["scales"], q["qzeros"], group, _sym)
            q["snr_db_f32"] = snr.snr_db(w, d)
            return q
        monkeypatch.setattr(gq, name, fp16_snr)
    _fails(tg.test_page_in_function_snr_closed_form)


def test_gptq_page_snr_per_column_caught(monkeypatch):
    """Norms taken per output column (SNRs averaged) instead of over the whole tensor."""
    def per_column(wt, deq):
        num = np.sqrt(np.sum(wt.astype(np.float64) ** 2, axis=0))
        den = np.maximum(np.sqrt(np.sum((wt - deq).astype(np.float64) ** 2, axis=0)), 1e-12)
        live = num > 0
        return float(np.mean(20.0 * np.log10(num[live] / den[live])))
    monkeypatch.setattr(gq, "_snr_page", per_column)
    _fails(tg.test_page_in_function_snr_closed_form)


def test_gptq_group_order_unstable_caught(monkeypatch):
    """Group order with the channels of a group reversed (an unstable sort)."""
    orig = gq.group_order
    def reversed_within(qweight, g_idx, group):
        qw, perm = orig(qweight, g_idx, group)
        perm = perm.reshape(-1, group)[:, ::-1].reshape(-1).copy()
        codes = gq.unpack_int32(qweight, 0)
        return gq.pack_int32(codes[perm], 0), perm
    monkeypatch.setattr(gq, "group_order", reversed_within)
    _fails(tg.test_group_order_bruteforce, True)


def test_gptq_group_order_inverse_perm_caught(monkeypatch):
    """Group order that gathers the codes by the inverse permutation."""
    orig = gq.group_order
    def inverse(qweight, g_idx, group):
        qw, perm = orig(qweight, g_idx, group)
        inv = np.argsort(perm).astype(np.int32)
        codes = gq.unpack_int32(qweight, 0)
        return gq.pack_int32(codes[inv], 0), perm
    monkeypatch.setattr(gq, "group_order", inverse)
    _fails(tg.test_group_order_bruteforce, False)
