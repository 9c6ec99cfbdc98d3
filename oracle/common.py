"""Scalar conventions shared by the oracle's modules (test infrastructure only)."""
from __future__ import annotations

import numpy as np


def sign_pm1(v: np.ndarray) -> np.ndarray:
    """Binarization sign: +1 where v >= 0, -1 otherwise (int8).

    [BitNet] §2.1 fixes the tie: zero maps to +1 (unlike numpy/torch sign,
    which returns 0 there and would make a ternary value).  -0.0 >= 0 holds,
    so negative zero also maps to +1.
    """
    v = np.asarray(v)
    return np.where(v >= 0, 1, -1).astype(np.int8)


def to_f16(a) -> np.ndarray:
    """Round (from fp64 or fp32) to IEEE half, round-half-to-even."""
    return np.asarray(a, dtype=np.float64).astype(np.float16)


def f16_bits(a16: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a16, dtype=np.float16).view(np.uint16)


def f16_from_bits(b: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
