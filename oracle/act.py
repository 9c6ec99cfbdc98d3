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

Arbitrary activation bit widths ([ABQ] §1: any WnAm, e.g. W4A4, W6A6): with
m bits the symmetric range is [-Qm, Qm], Qm = 2^(m-1) - 1, and the same steps
run with Qm in place of 127 (m = 8 is the int8 quantizer above).  The
codes still fit a two's-complement byte whose bits m-1..7 all equal the
sign, so the m-bit product needs only planes 0..m-2 and the sign plane 7
(weight -2^(m-1)).
"""
from __future__ import annotations

import numpy as np

from . import bitserial


def qmax(bits: int) -> int:
    """Largest code of the symmetric m-bit range: 2^(m-1) - 1."""
    assert 2 <= bits <= 8
    return (1 << (bits - 1)) - 1


def quantize(x_f32: np.ndarray, bits: int = 8):
    """x_f32: [M, K] float32.  Returns (q int8 [M,K], d float32 [M]) with
    q in [-Qm, Qm], Qm = 2^(bits-1) - 1 (127 for the default 8 bits)."""
    x = np.asarray(x_f32, dtype=np.float32)
    assert x.ndim == 2
    Q = qmax(bits)
    Qf = np.float32(Q)
    amax = np.max(np.abs(x), axis=1)                       # float32, exact
    M, K = x.shape
    q = np.zeros((M, K), dtype=np.int8)
    d = np.zeros(M, dtype=np.float32)
    for m in range(M):
        a = amax[m]
        if a == 0:
            continue
        s = Qf / a                                         # fl32 division
        prod = x[m] * s                                    # fl32 multiply
        q[m] = np.clip(np.rint(prod), -Q, Q).astype(np.int8)
        d[m] = a / Qf
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


def binarize(x_f32: np.ndarray):
    """Binary activations of the fully binary path ([BitNet] §2.1 sign with
    the tie at 0 going to +1; §2.3 XNOR+popcount product): x_b = sign(x) in
    {-1, +1} and a per-token scale beta = mean_k |x_k| (fp64; the page gives
    only the weight scale, beta is the reading taken so that beta * x_b
    approximates x).  Returns (x_b int8 [M, K], beta float64 [M])."""
    x = np.asarray(x_f32, dtype=np.float32)
    assert x.ndim == 2
    xb = np.where(x >= 0, 1, -1).astype(np.int8)           # -0.0 >= 0: +1
    beta = np.abs(x.astype(np.float64)).mean(axis=1)
    return xb, beta


def binary_words(xb: np.ndarray, Kp: int | None = None) -> np.ndarray:
    """Sign bits packed LSB first (1 <-> +1), zero bits past K up to Kp:
    [M, Kp/32] uint32."""
    M, K = xb.shape
    Kp = K if Kp is None else Kp
    bits = np.zeros((M, Kp), dtype=np.uint8)
    bits[:, :K] = (np.asarray(xb) > 0)
    return bitserial.pack_bits(bits)
