"""Affine uintx oracle, 2..7 bits (test infrastructure only).

Follows page uintx_quant.py (module docstring; _pack_shard, _unpack_shard, pack_uintx,
unpack_uintx; UIntXQuantizer.can_quantize, _quantize_impl, _dequantize_native).
The weight is bfloat16 and every arithmetic op is a bfloat16 tensor op, i.e. one
float32 op whose result is rounded to bfloat16 (bf16_round below).

Step list per group of G (64) consecutive weights along K, qmax = 2**nbits - 1:
  min, max over the group (exact)
  mn = min(min, 0), mx = max(max, 0)                    (preserve_zero)
  scale = bf(bf(mx - mn) / qmax); scale = max(scale, 2**-23)
  zp = clamp(0 - rint(bf(mn / scale)), 0, qmax)        -> int
  inv = bf(1 / scale)                                    (reciprocal first, as torch
                                                          evaluates 1.0 / tensor)
  q = clamp(bf(rint(bf(w * inv)) + zp), 0, qmax)        -> uint8
Dequantize: bf(bf(q - zp) * scale).
"""
from __future__ import annotations

import numpy as np

from ._fp import bf16_round as bf, f32, is_bf16

EPS = np.float32(np.finfo(np.float32).eps)   # 2**-23, exactly a bfloat16 too
SHARD_WIDTHS = (8, 4, 2, 1)                  # the page's shard order


def shard_widths(nbits: int):
    """Shard widths present in nbits, in pack order; bits [off, off + k) of a code go
    to the k-bit shard, off counted up from 0 in that order."""
    return [k for k in SHARD_WIDTHS if nbits & k]


def shard_nbytes(numel: int, k: int) -> int:
    vpb = 8 // k
    return -(-numel // vpb)


def packed_nbytes(numel: int, nbits: int) -> int:
    return sum(shard_nbytes(numel, k) for k in shard_widths(nbits))


def can_quantize(nbits: int, shape, group: int = 64) -> bool:
    """uint8 is refused (it was always left unquantized), as are non-2-D weights and
    K not divisible by the group size."""
    if nbits == 8 or not (2 <= nbits <= 8):
        return False
    if len(shape) != 2:
        return False
    return shape[1] % group == 0


def _pack_shard(vals: np.ndarray, k: int) -> np.ndarray:
    """Flat values < 2**k -> bytes, 8 // k per byte, planar: pad with zeros to a
    multiple of vpb, view as [vpb, L]; byte i = OR_j chunk_j[i] << (j * k)."""
    vpb = 8 // k
    if vpb == 1:
        return vals.copy()
    pad = (-vals.size) % vpb
    if pad:
        vals = np.concatenate([vals, np.zeros(pad, np.uint8)])
    chunks = vals.reshape(vpb, -1)
    out = chunks[0].copy()
    for j in range(1, vpb):
        out |= (chunks[j] << (j * k)).astype(np.uint8)
    return out


def _unpack_shard(packed: np.ndarray, k: int, numel: int) -> np.ndarray:
    vpb = 8 // k
    if vpb == 1:
        return packed[:numel].copy()
    out = np.empty((vpb, packed.size), np.uint8)
    for j in range(vpb):
        out[j] = (packed >> (j * k)) & ((1 << k) - 1)
    return out.reshape(-1)[:numel]


def pack(codes, nbits: int) -> np.ndarray:
    """Codes (values < 2**nbits) -> one flat uint8 buffer: the shards in pack order,
    concatenated."""
    flat = np.asarray(codes).reshape(-1).astype(np.uint8)
    assert np.all(flat < (1 << nbits))
    shards, off = [], 0
    for k in shard_widths(nbits):
        shards.append(_pack_shard(((flat >> off) & ((1 << k) - 1)).astype(np.uint8), k))
        off += k
    return np.concatenate(shards) if len(shards) > 1 else shards[0]


def unpack(packed, nbits: int, numel: int) -> np.ndarray:
    """Inverse of pack -> flat uint8 [numel]."""
    packed = np.asarray(packed, np.uint8)
    out = np.zeros(numel, np.uint8)
    off = pos = 0
    for k in shard_widths(nbits):
        nb = shard_nbytes(numel, k)
        out |= (_unpack_shard(packed[pos:pos + nb], k, numel) << off).astype(np.uint8)
        off += k
        pos += nb
    assert pos == packed.size
    return out


def quantize(w, nbits: int, group: int = 64):
    """bf16 [N, K] (as float32 values) -> dict(packed uint8 flat, scale bf16 as float32
    [N, K/G], scale_bytes uint8 [N, 2K/G] little-endian, zero_point uint8 [N, K/G],
    codes uint8 [N, K])."""
    x = f32(w)
    assert can_quantize(nbits, x.shape, group), (nbits, x.shape, group)
    assert is_bf16(x), "uintx arithmetic is specified for bfloat16 weights"
    qmin, qmax = 0, (1 << nbits) - 1
    n, k = x.shape
    wv = x.reshape(n, k // group, group)
    mn = wv.min(axis=2)
    mx = wv.max(axis=2)
    mn_neg = np.minimum(mn, np.float32(0.0))
    mx_pos = np.maximum(mx, np.float32(0.0))
    scale = bf(bf(mx_pos - mn_neg) / np.float32(qmax - qmin))
    scale = np.maximum(scale, EPS)
    zp = bf(np.float32(qmin) - np.rint(bf(mn_neg / scale)))
    zp = np.clip(zp, qmin, qmax).astype(np.int32)
    inv = bf(np.float32(1.0) / scale)
    t = bf(wv * inv[:, :, None])
    q = bf(np.rint(t) + zp[:, :, None].astype(np.float32))
    q = np.clip(q, qmin, qmax).astype(np.uint8).reshape(n, k)
    sbits = (scale.view(np.uint32) >> 16).astype(np.uint16)
    return dict(
        packed=pack(q, nbits),
        scale=scale,
        scale_bytes=np.ascontiguousarray(sbits.astype("<u2")).view(np.uint8).reshape(n, 2 * (k // group)),
        zero_point=zp.astype(np.uint8),
        codes=q,
    )


def scale_from_bytes(scale_bytes, n: int, groups: int) -> np.ndarray:
    u = np.ascontiguousarray(scale_bytes, np.uint8).view("<u2").reshape(n, groups)
    return (u.astype(np.uint32) << 16).view(np.float32)


def dequantize(packed, scale_bytes, zero_point, nbits: int, n: int, k: int, group: int = 64) -> np.ndarray:
    """-> bf16 values as float32 [N, K]: bf(bf(q - zp) * scale)."""
    q = unpack(packed, nbits, n * k).reshape(n, k // group, group).astype(np.float32)
    scale = scale_from_bytes(scale_bytes, n, k // group)
    zp = np.asarray(zero_point, np.uint8).reshape(n, k // group).astype(np.float32)
    dq = bf(q - zp[:, :, None])
    dq = bf(dq * scale[:, :, None])
    return dq.reshape(n, k)


def bits_per_weight(nbits: int, group: int = 64) -> float:
    """nbits per code plus a 16-bit scale and an 8-bit zero point per group."""
    return nbits + (16 + 8) / group
