"""Storage formats of the oracle: bf16 and fp32 rounding points.

Test infrastructure only: nothing in the GPU library imports this module.

Every rounding point of the layer is "compute in fp64, hold the value in
fp32 (the accumulator type), then store it as bf16 with round-to-nearest-even".
The pages name bf16 and MXFP8 as the layer's precisions (kucoin.com news flash
"O MoK do Cursor alcança aumento de desempenho de 2,37x no NVIDIA GB300
NVL72", section 03) but fix no rounding points; the points used here are
listed with the other readings of the pages in the design notes.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) exactly: a bf16 is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f32(v) -> np.ndarray:
    """Round to fp32 (nearest, ties to even) and return the value as fp64."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_bits(v) -> np.ndarray:
    """Round to fp32, then to bf16 (each nearest, ties to even); return bits."""
    a = np.asarray(v, dtype=np.float64).astype(np.float32)
    if not np.all(np.isfinite(a)):
        raise FloatingPointError("bf16_bits: non-finite value")
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def bf16(v) -> np.ndarray:
    """Value of ``v`` after the bf16 rounding point (fp64 array)."""
    return bf16_to_f64(bf16_bits(v))


def identity(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float64)
