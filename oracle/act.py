"""Per-token int8 activation quantizer (test infrastructure only).

[HGF] §1.2: activations are quantized to 8-bit integers and the integer
product is rescaled by gamma_x * gamma_W / 127, i.e. per-token absmax scaling
to the symmetric range [-127, 127].  [BVSR] (introduction) converts the input
activations online into its bit format before the AND+popcount GEMV.

The pages fix only "int8" and "/127".  The order of operations and the
rounding below are the reading taken, chosen so that a float32 emulation here
and a float32 GPU kernel agree bit for bit:

    amax = max_k |x_k|                       (float32, exact)
    amax == 0  ->  q = 0, d = 0
    s = fl32(127 / amax)                     (correctly rounded division)
    q_k = clamp(rint(fl32(x_k * s)), -127, 127)   (round half to even)
    d = fl32(amax / 127)                     (dequantization step)

Then x_hat_k = q_k * d is the activation the integer paths multiply.
Group sums S[g] = sum_{k in g} q_k feed the zero-point and offset terms.
"""
from __future__ import annotations

import numpy as np

from . import bitserial


def quantize(x_f32: np.ndarray):
    """x_f32: [M, K] float32.  Returns (q int8 [M,K], d float32 [M])."""
    x = np.asarray(x_f32, dtype=np.float32)
    assert x.ndim == 2
    amax = np.max(np.abs(x), axis=1)                       # float32, exact
    M, K = x.shape
    q = np.zeros((M, K), dtype=np.int8)
    d = np.zeros(M, dtype=np.float32)
    for m in range(M):
        a = amax[m]
        if a == 0:
            continue
        s = np.float32(127.0) / a                          # fl32 division
        prod = x[m] * s                                    # fl32 multiply
        q[m] = np.clip(np.rint(prod), -127, 127).astype(np.int8)
        d[m] = a / np.float32(127.0)
    return q, d


def group_sums(q: np.ndarray, group: int) -> np.ndarray:
    """S[m, g] = sum of q over the g-th run of `group` consecutive channels."""
    q = np.asarray(q, dtype=np.int64)
    M, K = q.shape
    assert K % group == 0
    return q.reshape(M, K // group, group).sum(axis=-1)


def planes(q: np.ndarray) -> np.ndarray:
    """Activation bit-planes packed as words: [8, M, K/32] uint32 (plane j =
    bit j of the two's-complement byte, bit i of word w <-> channel 32w+i)."""
    return bitserial.pack_bits(bitserial.act_planes(q))
