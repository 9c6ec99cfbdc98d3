"""Bit-planes and the AND+popcount contraction (test infrastructure only).

[ABQ] (abstract, §1) rebuilds an arbitrary-bit integer matrix product from
binary operations (its "BTC-equivalent" engine); [BVSR] (introduction)
contracts bitvectors with online-quantized activations by bitwise AND and
population count, without dequantizing.  Both rest on the identity

    sum_k qw[k] * qx[k] = sum_i sum_j  u_i * v_j * popcount(W_i AND X_j)

where qw = sum_i u_i W_i and qx = sum_j v_j X_j are decompositions of the two
integer operands into {0,1} bit-planes W_i, X_j with integer plane weights
u_i, v_j.  This module writes those steps out literally; the oracle's GEMV
(oracle/gemv.py) uses a plain int64 dot product instead, and the tests pin the
two against each other.

Activation planes: two's complement of the int8 value, X_j = bit j of
uint8(q), with plane weights v_j = 2^j for j < 7 and v_7 = -128.  The pages
only say "8 planes combined by AND+popcount"; this is the reading taken (an
offset-binary split would give the same integer).
"""
from __future__ import annotations

import numpy as np

ACT_PLANE_WEIGHTS = np.array([1, 2, 4, 8, 16, 32, 64, -128], dtype=np.int64)


def act_plane_weights(bits: int) -> np.ndarray:
    """Plane weights for m-bit codes q in [-(2^(m-1)-1), 2^(m-1)-1] stored as
    int8: bits m-1..7 of the byte all equal the sign, so q is planes 0..m-2
    with weights 2^j plus the sign plane 7 with weight -2^(m-1); planes
    m-1..6 get weight 0.  bits = 8 gives ACT_PLANE_WEIGHTS."""
    assert 2 <= bits <= 8
    w = np.zeros(8, dtype=np.int64)
    for j in range(bits - 1):
        w[j] = 1 << j
    w[7] = -(1 << (bits - 1))
    return w


def act_planes(q: np.ndarray) -> np.ndarray:
    """Two's-complement bit-planes of int8 values: out[j] = bit j of uint8(q)."""
    u = np.asarray(q, dtype=np.int8).view(np.uint8).astype(np.int64)
    return np.stack([(u >> j) & 1 for j in range(8)]).astype(np.uint8)


def unsigned_planes(qw: np.ndarray, nbits: int) -> np.ndarray:
    """Planes of an unsigned code: out[i] = bit i of qw (plane weight 2^i)."""
    u = np.asarray(qw).astype(np.int64)
    return np.stack([(u >> i) & 1 for i in range(nbits)]).astype(np.uint8)


def pack_bits(bits: np.ndarray) -> np.ndarray:
    """Pack {0,1} values along the last axis into uint32 words, LSB first:
    bit i of word w holds element 32*w + i.  The last axis must be a multiple
    of 32."""
    bits = np.asarray(bits, dtype=np.uint64)
    K = bits.shape[-1]
    assert K % 32 == 0
    b = bits.reshape(bits.shape[:-1] + (K // 32, 32))
    shifts = np.arange(32, dtype=np.uint64)
    return (b << shifts).sum(axis=-1).astype(np.uint32)


def unpack_bits(words: np.ndarray) -> np.ndarray:
    """Inverse of pack_bits."""
    w = np.asarray(words, dtype=np.uint32).astype(np.uint64)
    shifts = np.arange(32, dtype=np.uint64)
    b = (w[..., None] >> shifts) & 1
    return b.reshape(w.shape[:-1] + (w.shape[-1] * 32,)).astype(np.uint8)


def popcount(words: np.ndarray) -> np.ndarray:
    return np.bitwise_count(np.asarray(words, dtype=np.uint32)).astype(np.int64)


def and_popcount_dot(w_words: np.ndarray, w_weights, x_words: np.ndarray, x_weights,
                     group_words: int | None = None) -> np.ndarray:
    """AND+popcount contraction of packed planes.

    w_words: [I, N, Kw] uint32 weight planes; w_weights: I integer plane weights
    x_words: [J, M, Kw] uint32 activation planes; x_weights: J plane weights
    group_words: if given, partial sums are kept per group of that many words.

    Returns int64 [M, N] (or [M, N, Kw // group_words]) equal to
    sum_i sum_j u_i v_j popcount(W_i AND X_j), summed over the words.
    """
    w_words = np.asarray(w_words, dtype=np.uint32)
    x_words = np.asarray(x_words, dtype=np.uint32)
    I, N, Kw = w_words.shape
    J, M, Kw2 = x_words.shape
    assert Kw == Kw2
    g = Kw if group_words is None else group_words
    assert Kw % g == 0
    G = Kw // g
    out = np.zeros((M, N, G), dtype=np.int64)
    for i in range(I):
        for j in range(J):
            both = w_words[i][None, :, :] & x_words[j][:, None, :]       # [M, N, Kw]
            pc = popcount(both).reshape(M, N, G, g).sum(axis=-1)
            out += int(w_weights[i]) * int(x_weights[j]) * pc
    return out[..., 0] if group_words is None else out


def xnor_popcount_dot(b_words: np.ndarray, s_words: np.ndarray, K: int) -> np.ndarray:
    """Dot product of two +-1 vectors given as packed sign bits (1 <-> +1).

    [BitNet] §2.3 writes the binary product as popcount(xnor(a, b)) times a
    scale, leaving out the affine map; the exact value is
        sum_k a_k b_k = (#agreements) - (#disagreements) = K - 2*popcount(a XOR b).
    b_words: [N, Kw], s_words: [Kw] for one vector; returns int64 [N].
    """
    x = np.asarray(b_words, dtype=np.uint32) ^ np.asarray(s_words, dtype=np.uint32)[None, :]
    return K - 2 * popcount(x).sum(axis=-1)
