"""Seeded synthetic weight matrices and activation statistics.

These are the only inputs shared by the CPU oracle and the HIP path. Nothing here
implements any step of the quantization method: values are drawn with numpy's PCG64
generator in float32 and, for bf16 workloads, rounded to bfloat16 by torch's own
float32 -> bfloat16 conversion (round to nearest, ties to even).

The shapes and distributions stand in for the pages' weights, which are not
available: a 4-bit GPTQ export of a small decoder (export_gptq_cpu.py), the
gate_up projection [34816, 5120] of a speculative-decoding drafter
(quantize_dflash_mxfp4.py, docstring of quantize_mxfp4) and base models quantized
with affine uintx (uintx_quant.py).

Every generator returns CPU tensors; callers move them to the GPU.
"""
from __future__ import annotations

import numpy as np
import torch

__all__ = [
    "normal_weight", "gptq_sym_weight", "gptq_asym_weight", "mxfp4_weight",
    "uintx_weight", "awq_activation_stat", "adversarial_weight",
    "WORKLOADS",
]


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _finish(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(dtype) if dtype != torch.float32 else t


def normal_weight(n: int, k: int, seed: int, std: float = 0.02,
                  dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """[n, k] entries N(0, std)."""
    x = _rng(seed).standard_normal((n, k), dtype=np.float32) * np.float32(std)
    return _finish(x, dtype)


def gptq_sym_weight(n: int = 256, k: int = 1024, seed: int = 1) -> torch.Tensor:
    """float32 [n, k], N(0, 0.02)."""
    return normal_weight(n, k, seed, 0.02, torch.float32)


def gptq_asym_weight(n: int = 4096, k: int = 4096, seed: int = 2,
                     outlier_frac: float = 0.01, outlier_gain: float = 20.0) -> torch.Tensor:
    """bf16 [n, k], N(0, 0.02) with round(outlier_frac * k) distinct input columns
    scaled by outlier_gain before the bf16 rounding."""
    rng = _rng(seed)
    x = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    cols = rng.choice(k, size=int(round(outlier_frac * k)), replace=False)
    x[:, cols] *= np.float32(outlier_gain)
    return _finish(x, torch.bfloat16)


def mxfp4_weight(n: int = 34816, k: int = 5120, seed: int = 3,
                 dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """[n, k], N(0, 0.015) times a per-row gain drawn lognormal(0, 0.5)."""
    rng = _rng(seed)
    gain = rng.lognormal(0.0, 0.5, size=(n, 1)).astype(np.float32)
    x = rng.standard_normal((n, k), dtype=np.float32)
    x *= np.float32(0.015)
    x *= gain
    return _finish(x, dtype)


def uintx_weight(n: int = 3072, k: int = 12288, seed: int = 4,
                 outlier_frac: float = 0.001, dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """[n, k] (bf16 by default), N(0, 0.02) with round(outlier_frac * n * k) distinct
    entries replaced by U(-0.5, 0.5)."""
    rng = _rng(seed)
    x = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    m = int(round(outlier_frac * n * k))
    if m:
        idx = rng.choice(n * k, size=m, replace=False)
        x.reshape(-1)[idx] = rng.uniform(-0.5, 0.5, size=m).astype(np.float32)
    return _finish(x, dtype)


def awq_activation_stat(k: int = 5120, seed: int = 5) -> torch.Tensor:
    """float32 [k] per-input-channel mean |x| stand-in, lognormal(0, 1)."""
    return torch.from_numpy(_rng(seed).lognormal(0.0, 1.0, size=k).astype(np.float32))


# Block kinds used by adversarial_weight. Each kind fills one 128-wide span of a row
# (a multiple of every group size used here: 32, 64, 128).
_ADV_KINDS = (
    "normal", "zeros", "signed_zeros", "constant", "pow2_max", "half_steps",
    "subnormal", "below_pow2", "huge", "tiny_mixed", "sparse_outlier", "all_negative",
)


def adversarial_weight(n: int, k: int, seed: int = 6,
                       dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """[n, k] with k % 128 == 0. Each 128-wide span of each row is one of the kinds
    in _ADV_KINDS, chosen at random: all zeros, +-0.0 mixes, constant spans, spans
    whose magnitude maximum is an exact power of two, spans made of multiples of
    power-of-two half steps (exact ties for every rounding grid used here),
    bfloat16/float32 subnormals, maxima one float32 ulp below a power of two, very
    large and very small magnitudes, a lone outlier, and all-negative spans. For
    float16 the very large, subnormal and very small kinds use float16's own range
    (2**12 scale, multiples of 2**-24, 2**-24..2**-15), with the same random draws."""
    assert k % 128 == 0
    rng = _rng(seed)
    half = dtype == torch.float16
    huge_e, sub_e, tiny_lo, tiny_hi = (12, -24, -24, -14) if half else (100, -133, -126, -100)
    x = np.empty((n, k), dtype=np.float32)
    spans = x.reshape(n, k // 128, 128)
    kinds = rng.integers(0, len(_ADV_KINDS), size=(n, k // 128))
    for r in range(n):
        for c in range(k // 128):
            kind = _ADV_KINDS[kinds[r, c]]
            e = int(rng.integers(-20, 6))
            if kind == "normal":
                v = rng.standard_normal(128).astype(np.float32) * np.float32(2.0 ** e)
            elif kind == "zeros":
                v = np.zeros(128, np.float32)
            elif kind == "signed_zeros":
                v = np.where(rng.random(128) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
            elif kind == "constant":
                v = np.full(128, np.float32(rng.choice([-1.0, 1.0]) * 1.375 * 2.0 ** e), np.float32)
            elif kind == "pow2_max":
                v = (rng.uniform(-1, 1, 128) * 2.0 ** e).astype(np.float32)
                v[rng.integers(0, 128)] = np.float32(rng.choice([-1.0, 1.0]) * 2.0 ** e)
            elif kind == "half_steps":
                # integer multiples of 2**(e-4): many exact midpoints of coarse grids
                v = (rng.integers(-96, 97, 128).astype(np.float32) * np.float32(2.0 ** (e - 4)))
            elif kind == "subnormal":
                v = (rng.integers(-127, 128, 128).astype(np.float32) * np.float32(2.0 ** sub_e))
            elif kind == "below_pow2":
                v = (rng.uniform(-1, 1, 128) * 2.0 ** e).astype(np.float32)
                v[rng.integers(0, 128)] = np.nextafter(np.float32(2.0 ** e), np.float32(0))
            elif kind == "huge":
                v = (rng.standard_normal(128) * 2.0 ** huge_e).astype(np.float32)
            elif kind == "tiny_mixed":
                v = (rng.standard_normal(128) * 2.0 ** rng.integers(tiny_lo, tiny_hi, 128)).astype(np.float32)
            elif kind == "sparse_outlier":
                v = (rng.standard_normal(128) * 2.0 ** (e - 8)).astype(np.float32)
                v[rng.integers(0, 128)] = np.float32(rng.choice([-1.0, 1.0]) * 2.0 ** e * 3.1)
            else:  # all_negative
                v = -np.abs(rng.standard_normal(128).astype(np.float32)) * np.float32(2.0 ** e) - np.float32(2.0 ** (e - 2))
            spans[r, c] = v
    return _finish(x, dtype)


# The five workload configurations (sizes, dtype, recipe) by name.
WORKLOADS = {
    "gptq_sym_fp32_256x1024_g128": dict(fmt="gptq_sym", group=128, make=lambda: gptq_sym_weight()),
    "gptq_asym_bf16_4096x4096_g128": dict(fmt="gptq_asym", group=128, make=lambda: gptq_asym_weight()),
    "mxfp4_bf16_34816x5120": dict(fmt="mxfp4", group=32, make=lambda: mxfp4_weight()),
    "uintx_bf16_3072x12288_g64": dict(fmt="uintx", group=64, make=lambda: uintx_weight()),
    "awq_mxfp4_2048of34816x5120": dict(fmt="awq", group=32,
                                       make=lambda: (mxfp4_weight(), awq_activation_stat())),
}
