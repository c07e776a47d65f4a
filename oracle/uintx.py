"""Affine uintx oracle, 2..7 bits (test infrastructure only).

Follows page uintx_quant.py (module docstring; _pack_shard, _unpack_shard, pack_uintx,
unpack_uintx; UIntXQuantizer.can_quantize, _quantize_impl, _dequantize_native).
The arithmetic runs in the weight's own dtype (the page's docstring: usually
bfloat16): every op is one float32 op whose result is rounded to that dtype — bfloat16
or float16 (RNE, as torch's half ops compute in float32 and round) — or a plain float32
op for float32 weights. The scale is stored as the bytes of that dtype.
Reading for float32 weights: `scale / qmax` is the division the page writes (IEEE);
torch's GPU path multiplies by the float32 reciprocal instead, which changes the last
bit of about a third of the scales. For bfloat16 and float16 the two agree after the
rounding for every value (exhaustive check in the pins).
Reading for float16 weights: a group whose scale is below about 2**-16 has an infinite
float16 reciprocal, so w * inv is +inf, -inf or (for a zero weight) NaN; the clamp sends
the infinities to qmax and 0, and the NaN becomes code 0, which is what torch's float to
uint8 conversion returns for it on the CPU.

Step list per group of G (64 by default; 32 and 128 too) consecutive weights along K,
qmax = 2**nbits - 1, bf = rounding to the weight dtype:
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

EPS = np.float32(np.finfo(np.float32).eps)   # 2**-23, exactly a bfloat16 and a float16 too
DTYPES = ("bf16", "f16", "f32")
SCALE_BYTES = {"bf16": 2, "f16": 2, "f32": 4}


def f16(x) -> np.ndarray:
    """Round float32 values to float16 (RNE, gradual underflow, overflow to inf), back
    as float32."""
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float32)


def rounder(dtype: str):
    return {"bf16": bf, "f16": f16, "f32": lambda v: np.asarray(v, np.float32)}[dtype]


def is_dtype(x, dtype: str) -> bool:
    x = np.asarray(x, np.float32)
    return bool(np.array_equal(rounder(dtype)(x), x) or np.isnan(x).any())


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


def quantize(w, nbits: int, group: int = 64, dtype: str = "bf16"):
    """[N, K] weights of `dtype` (as float32 values) -> dict(packed uint8 flat, scale as
    float32 [N, K/G], scale_bytes uint8 [N, bytes * K/G] little-endian, zero_point uint8
    [N, K/G], codes uint8 [N, K])."""
    x = f32(w)
    rnd = rounder(dtype)
    assert can_quantize(nbits, x.shape, group), (nbits, x.shape, group)
    assert is_dtype(x, dtype), f"weights are not {dtype} values"
    qmin, qmax = 0, (1 << nbits) - 1
    n, k = x.shape
    wv = x.reshape(n, k // group, group)
    mn = wv.min(axis=2)
    mx = wv.max(axis=2)
    mn_neg = np.minimum(mn, np.float32(0.0))
    mx_pos = np.maximum(mx, np.float32(0.0))
    with np.errstate(over="ignore"):
        scale = rnd(rnd(mx_pos - mn_neg) / np.float32(qmax - qmin))
        scale = np.maximum(scale, EPS)
        zp = rnd(np.float32(qmin) - np.rint(rnd(mn_neg / scale)))
        zp = np.clip(zp, qmin, qmax).astype(np.int32)
        inv = rnd(np.float32(1.0) / scale)
    with np.errstate(invalid="ignore", over="ignore"):
        t = rnd(wv * inv[:, :, None])
        q = rnd(np.rint(t) + zp[:, :, None].astype(np.float32))
        q = np.clip(q, qmin, qmax)
    q = np.where(np.isnan(q), np.float32(0.0), q)     # 0 * inf (float16 only)
    q = q.astype(np.uint8).reshape(n, k)
    return dict(
        packed=pack(q, nbits),
        scale=scale,
        scale_bytes=scale_to_bytes(scale, dtype),
        zero_point=zp.astype(np.uint8),
        codes=q,
    )


def scale_to_bytes(scale, dtype: str = "bf16") -> np.ndarray:
    scale = np.ascontiguousarray(scale, np.float32)
    n = scale.shape[0]
    if dtype == "bf16":
        u = (scale.view(np.uint32) >> 16).astype("<u2")
    elif dtype == "f16":
        u = scale.astype("<f2")
    else:
        u = scale.astype("<f4")
    return np.ascontiguousarray(u).view(np.uint8).reshape(n, -1)


def scale_from_bytes(scale_bytes, n: int, groups: int, dtype: str = "bf16") -> np.ndarray:
    b = np.ascontiguousarray(scale_bytes, np.uint8)
    if dtype == "bf16":
        u = b.view("<u2").reshape(n, groups)
        return (u.astype(np.uint32) << 16).view(np.float32)
    if dtype == "f16":
        return b.view("<f2").reshape(n, groups).astype(np.float32)
    return b.view("<f4").reshape(n, groups).astype(np.float32)


def dequantize(packed, scale_bytes, zero_point, nbits: int, n: int, k: int, group: int = 64,
               dtype: str = "bf16") -> np.ndarray:
    """-> values of `dtype` as float32 [N, K]: rnd(rnd(q - zp) * scale)."""
    rnd = rounder(dtype)
    q = unpack(packed, nbits, n * k).reshape(n, k // group, group).astype(np.float32)
    scale = scale_from_bytes(scale_bytes, n, k // group, dtype)
    zp = np.asarray(zero_point, np.uint8).reshape(n, k // group).astype(np.float32)
    dq = rnd(q - zp[:, :, None])
    dq = rnd(dq * scale[:, :, None])
    return dq.reshape(n, k)


def bits_per_weight(nbits: int, group: int = 64, dtype: str = "bf16") -> float:
    """nbits per code plus a scale of the weight dtype and an 8-bit zero point per group."""
    return nbits + (8 * SCALE_BYTES[dtype] + 8) / group
