"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module only draws random numbers and converts them to the storage
dtypes the workloads use (fp32, bf16).  It contains none of the method's
arithmetic: no sign, no scale fit, no quantizer, no packing.  Both the CPU
oracle and the GPU library consume what it returns, so that the two sides see
bit-identical inputs.

Workloads (layer shapes are out x in, i.e. W is [N, K], x is [M, K]):

  sign    : W ~ N(0, 1)      fp32,  x ~ N(0, 1) fp32,  256 x 256, M = 1
  rabit   : W ~ N(0, 0.02^2) fp32,  x ~ N(0, 1) -> bf16, Llama-2-7B shapes
  ternary : W ~ N(0, 0.02^2) fp32,  x ~ N(0, 1) -> bf16, 512-dim 8-layer
            shapes and 4096 x 4096, M in {1, 16}
  w2a8    : W ~ N(0, 0.02^2) fp32,  x ~ N(0, 1) with 1% of the input
            channels scaled x20 (same channels for every token) -> bf16
  bvsr    : W ~ N(0, 0.015^2) fp32, x ~ N(0, 1) -> bf16, 70B-class shapes
  hgf     : the ternary workload plus a rank-r correction: A [K, r] and
            B [r, N] ~ N(0, 0.02^2) rounded to fp16, gate parameter 0.1

The pages measure on trained Llama/LLaMA/Gemma layers and text datasets; these
Gaussian layers of the same shapes stand in for them.
"""
from __future__ import annotations

import math

import numpy as np

# Workload table: (config id, name, weight sigma, shapes, token counts, x dtype)
CONFIGS = {
    "sign": dict(cfg=1, sigma=1.0, shapes=[(256, 256)], M=[1], x_dtype="f32"),
    "rabit": dict(cfg=2, sigma=0.02,
                  shapes=[(4096, 4096), (11008, 4096), (4096, 11008)],
                  M=[1], x_dtype="bf16"),
    "ternary": dict(cfg=3, sigma=0.02,
                    shapes=[(512, 512), (2048, 512), (512, 2048), (4096, 4096)],
                    M=[1, 16], x_dtype="bf16"),
    "w2a8": dict(cfg=4, sigma=0.02,
                 shapes=[(4096, 4096), (11008, 4096), (4096, 11008)],
                 M=[1, 4, 8, 16, 64], x_dtype="bf16"),
    "bvsr": dict(cfg=5, sigma=0.015,
                 shapes=[(8192, 8192), (28672, 8192)], M=[1], x_dtype="bf16"),
}

ROLE_W, ROLE_X, ROLE_OUTLIER, ROLE_LORA = 0, 1, 2, 3


def seed_for(cfg: int, shape_idx: int, role: int) -> int:
    """Seed of one random stream: 1000*cfg + 10*shape_idx + role."""
    return 1000 * cfg + 10 * shape_idx + role


def rng(cfg: int, shape_idx: int, role: int) -> np.random.Generator:
    return np.random.default_rng(seed_for(cfg, shape_idx, role))


def gaussian_f32(gen: np.random.Generator, shape, sigma: float) -> np.ndarray:
    """N(0, sigma^2) samples, drawn in float64 and stored as float32."""
    return (gen.standard_normal(shape) * sigma).astype(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-half-to-even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def weights(name: str, shape_idx: int, N: int, K: int, seed_offset: int = 0) -> np.ndarray:
    """fp32 weight matrix [N, K] for a workload (Gaussian, workload sigma)."""
    c = CONFIGS[name]
    gen = np.random.default_rng(seed_for(c["cfg"], shape_idx, ROLE_W) + 100000 * seed_offset)
    return gaussian_f32(gen, (N, K), c["sigma"])


def outlier_columns(name: str, shape_idx: int, K: int, frac: float = 0.01,
                    seed_offset: int = 0) -> np.ndarray:
    """ceil(frac*K) distinct input-channel indices, sorted (w2a8 outliers)."""
    c = CONFIGS[name]
    gen = np.random.default_rng(seed_for(c["cfg"], shape_idx, ROLE_OUTLIER) + 100000 * seed_offset)
    n = int(math.ceil(frac * K))
    return np.sort(gen.choice(K, size=n, replace=False)).astype(np.int64)


def activations(name: str, shape_idx: int, M: int, K: int, seed_offset: int = 0):
    """Activations for a workload.

    Returns (x_store, x_f32): x_store is what a caller hands to the library
    (float32 array for 'sign', uint16 bf16 bits otherwise) and x_f32 its exact
    float32 value.
    """
    c = CONFIGS[name]
    gen = np.random.default_rng(seed_for(c["cfg"], shape_idx, ROLE_X) + 100000 * seed_offset)
    x = gaussian_f32(gen, (M, K), 1.0)
    if name == "w2a8":
        cols = outlier_columns(name, shape_idx, K, seed_offset=seed_offset)
        x[:, cols] *= np.float32(20.0)
    if c["x_dtype"] == "f32":
        return x, x.copy()
    bits = f32_to_bf16_bits(x)
    return bits, bf16_bits_to_f32(bits)


def random_bf16(gen: np.random.Generator, shape, scale: float = 1.0):
    """Generic bf16 activations (bits, f32 value) for edge-case tests."""
    x = gaussian_f32(gen, shape, scale)
    bits = f32_to_bf16_bits(x)
    return bits, bf16_bits_to_f32(bits)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE half (round-half-to-even); returns uint16 bits."""
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32).astype(np.float16)).view(np.uint16)


def lora_params(shape_idx: int, N: int, K: int, r: int, sigma: float = 0.02,
                seed_offset: int = 0):
    """Low-rank correction parameters of an hgf layer (ternary config seeds).

    Returns (A_bits [K, r], B_bits [r, N]) as fp16 bit patterns and the gate
    parameter alpha (float32 0.1).  A and B are drawn N(0, sigma^2) in
    float64, stored float32, then rounded to fp16.
    """
    gen = np.random.default_rng(seed_for(CONFIGS["ternary"]["cfg"], shape_idx, ROLE_LORA)
                                + 100000 * seed_offset)
    A = gaussian_f32(gen, (K, r), sigma)
    B = gaussian_f32(gen, (r, N), sigma)
    return f32_to_f16_bits(A), f32_to_f16_bits(B), np.float32(0.1)
