"""4-bit GPTQ oracle (test infrastructure only).

Follows page export_gptq_cpu.py: pack_int32, quantize_sym (vLLM uint4b8: the weight
is (code - 8) * scale, code in [0, 15], zero points ignored — module docstring) and
quantize_asym (a real per-group zero point stored as itself, no minus one).

Layouts (GPTQ stores the transposed weight [K, N]):
  qweight int32 [K/8, N]   nibble i of word (r, n) = code of (k = 8r + i, n)
  qzeros  int32 [K/G, N/8] nibble i of word (g, q) = zero point of (g, n = 8q + i);
                           symmetric: every nibble 7; asymmetric: the zero point
  scales  fp16  [K/G, N]   the float32 group scale rounded to fp16 (RNE)
  g_idx   int32 [K]        k // G; act-order (quantize_act_order): the group of column k

Act-order (the "desc_act" field the page writes into its quantization_config as False,
and the g_idx tensor it stores): GPTQ checkpoints with desc_act true form the groups over
the input channels taken in a given order (by decreasing activation statistic) rather
than in index order, keep qweight in the original channel order, and record each
channel's group in g_idx; a consumer dequantizes channel k with the scale and zero point
of group g_idx[k]. Reading: the page's own per-group formulas (quantize_sym /
quantize_asym) applied to those groups.
"""
from __future__ import annotations

import numpy as np

from ._fp import f32

EPS_SCALE = np.float32(1e-9)   # the pages' clamp(min=1e-9), taken in float32


def pack_int32(codes, dim: int) -> np.ndarray:
    """Pack 8 nibbles per int32 along `dim` (0 or 1) of a 2-D array, lowest nibble
    first. Bits are built as uint32 and viewed as int32 (nibble 15 at i = 7 sets the
    sign bit)."""
    c = np.asarray(codes).astype(np.uint32)
    assert c.ndim == 2 and np.all(c < 16)
    if dim == 0:
        k, n = c.shape
        assert k % 8 == 0
        out = np.zeros((k // 8, n), np.uint32)
        for i in range(8):
            out |= c[i::8, :] << np.uint32(4 * i)
    else:
        k, n = c.shape
        assert n % 8 == 0
        out = np.zeros((k, n // 8), np.uint32)
        for i in range(8):
            out |= c[:, i::8] << np.uint32(4 * i)
    return out.view(np.int32)


def unpack_int32(words, dim: int) -> np.ndarray:
    """Inverse of pack_int32: -> uint8 nibbles."""
    u = np.ascontiguousarray(words).view(np.uint32)
    if dim == 0:
        k8, n = u.shape
        out = np.empty((k8 * 8, n), np.uint8)
        for i in range(8):
            out[i::8, :] = (u >> np.uint32(4 * i)) & 0xF
    else:
        k, n8 = u.shape
        out = np.empty((k, n8 * 8), np.uint8)
        for i in range(8):
            out[:, i::8] = (u >> np.uint32(4 * i)) & 0xF
    return out


def _groups(w, group: int):
    x = f32(w)
    assert x.ndim == 2
    n, k = x.shape
    assert k % group == 0 and k % 8 == 0 and n % 8 == 0, (n, k, group)
    wt = np.ascontiguousarray(x.T)                 # [K, N]
    return wt, wt.reshape(k // group, group, n), n, k


def quantize_sym(w, group: int = 128):
    """[N, K] -> dict(qweight, qzeros, scales, g_idx, codes [K, N], scale_f32 [G, N],
    snr_db_f32). Per (group, column): amax = max |x|; scale = max(amax / 8, 1e-9);
    code = clamp(rint(x / scale) + 8, 0, 15). snr_db_f32 is the page's in-function SNR,
    computed with the float32 (not the stored fp16) scale."""
    wt, blocks, n, k = _groups(w, group)
    g = k // group
    amax = np.abs(blocks).max(axis=1)                              # [G, N]
    scale = np.maximum(amax / np.float32(8.0), EPS_SCALE)          # float32
    codes = np.clip(np.rint(blocks / scale[:, None, :]) + np.float32(8.0), 0, 15)
    deq = ((codes - np.float32(8.0)) * scale[:, None, :]).reshape(k, n)
    codes = codes.reshape(k, n).astype(np.uint8)
    with np.errstate(over="ignore"):                    # scales past fp16's range round to inf
        scales16 = scale.astype(np.float16)
    return dict(
        qweight=pack_int32(codes, 0),
        qzeros=pack_int32(np.full((g, n), 7, np.uint8), 1),
        scales=scales16,
        g_idx=(np.arange(k, dtype=np.int32) // group).astype(np.int32),
        codes=codes, scale_f32=scale,
        snr_db_f32=_snr_page(wt, deq),
    )


def quantize_asym(w, group: int = 128):
    """[N, K] -> dict(qweight, qzeros, scales, g_idx, codes, zp [G, N], scale_f32,
    snr_db_f32). Per (group, column): scale = max(max - min, 1e-9) / 15;
    zp = clamp(rint(-min / scale), 0, 15); code = clamp(rint(x / scale) + zp, 0, 15)."""
    wt, blocks, n, k = _groups(w, group)
    wmax, wmin = blocks.max(axis=1), blocks.min(axis=1)
    scale = np.maximum(wmax - wmin, EPS_SCALE) / np.float32(15.0)
    zp = np.clip(np.rint(-wmin / scale), 0, 15)
    codes = np.clip(np.rint(blocks / scale[:, None, :]) + zp[:, None, :], 0, 15)
    deq = ((codes - zp[:, None, :]) * scale[:, None, :]).reshape(k, n)
    codes = codes.reshape(k, n).astype(np.uint8)
    zp = zp.astype(np.uint8)
    with np.errstate(over="ignore"):                    # scales past fp16's range round to inf
        scales16 = scale.astype(np.float16)
    return dict(
        qweight=pack_int32(codes, 0),
        qzeros=pack_int32(zp, 1),
        scales=scales16,
        g_idx=(np.arange(k, dtype=np.int32) // group).astype(np.int32),
        codes=codes, zp=zp, scale_f32=scale,
        snr_db_f32=_snr_page(wt, deq),
    )


def quantize_act_order(w, group: int, sym: bool, perm):
    """Act-order variant: group g = the columns perm[g*G : (g+1)*G] (perm a permutation of
    0..K-1). Scales and zero points [K/G, N] per such group as quantize_sym /
    quantize_asym compute them; codes and qweight in the original column order;
    g_idx[k] = the group of column k."""
    x = f32(w)
    k = x.shape[1]
    perm = np.asarray(perm, np.int64)
    assert perm.shape == (k,) and np.array_equal(np.sort(perm), np.arange(k)), "perm must be a permutation"
    q = (quantize_sym if sym else quantize_asym)(x[:, perm], group)   # groups over the permuted columns
    codes = np.empty_like(q["codes"])                                 # [K, N]: back to column order
    codes[perm] = q["codes"]
    g_idx = np.empty(k, np.int32)
    g_idx[perm] = (np.arange(k) // group).astype(np.int32)
    q.update(qweight=pack_int32(codes, 0), codes=codes, g_idx=g_idx)
    return q


def group_order(qweight, g_idx, group: int):
    """Act-order tensors rearranged into group order: the channels taken group by group,
    ascending channel index within a group (a stable sort by g_idx), so that group g's
    channels sit at positions g*G .. g*G + G - 1 and the index-order GPTQ layout (group
    k // G) applies once the activations are gathered the same way: x @ dequant^T is
    unchanged when column j of the rearranged weight meets x[perm[j]].
    Returns (qweight [K/8, N] with nibble i of word (r, n) = code of channel perm[8r + i],
    perm int32 [K] = the channel at each position). Every group must hold exactly G
    channels (as quantize_act_order makes them)."""
    codes = unpack_int32(qweight, 0)                                # [K, N]
    k = codes.shape[0]
    gi = np.asarray(g_idx, np.int64)
    assert gi.shape == (k,) and k % group == 0
    assert gi.min(initial=0) >= 0 and gi.max(initial=0) < k // group, "g_idx out of range"
    assert np.all(np.bincount(gi, minlength=k // group) == group), "every group needs exactly G channels"
    perm = np.argsort(gi, kind="stable")
    return pack_int32(codes[perm], 0), perm.astype(np.int32)


def _snr_page(wt, deq) -> float:
    """20 log10(||w|| / max(||w - deq||, 1e-12)) with float64 norms of float32 data."""
    num = np.sqrt(np.sum(wt.astype(np.float64) ** 2))
    den = max(np.sqrt(np.sum((wt - deq).astype(np.float64) ** 2)), 1e-12)
    with np.errstate(divide="ignore"):
        return float(20.0 * np.log10(num / den))


def dequantize(qweight, scales, qzeros, group: int, sym: bool, g_idx=None) -> np.ndarray:
    """Stored tensors -> float32 [N, K] (the caller's layout). Symmetric:
    (code - 8) * scale, qzeros ignored; asymmetric: (code - zp) * scale, zp read from
    qzeros. The scale is the stored fp16 value widened to float32. Column k uses group
    k // G, or g_idx[k] when g_idx is given (act-order)."""
    codes = unpack_int32(qweight, 0).astype(np.float32)            # [K, N]
    k, n = codes.shape
    s = np.asarray(scales, np.float16).astype(np.float32)           # [G, N]
    if sym:
        zp = np.full(s.shape, 8.0, np.float32)
    else:
        zp = unpack_int32(qzeros, 1).astype(np.float32)             # [G, N]
    gi = np.arange(k) // group if g_idx is None else np.asarray(g_idx, np.int64)
    with np.errstate(invalid="ignore"):                 # an inf scale times code - zp = 0: NaN
        d = (codes - zp[gi, :]) * s[gi, :]                          # row k uses group gi[k]
    return np.ascontiguousarray(d.T)


def bits_per_weight(group: int) -> float:
    """4 bits per code plus a 16-bit scale and a 4-bit zero point per group."""
    return 4 + (16 + 4) / group
