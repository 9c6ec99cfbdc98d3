"""Pins of the arbitrary-bit (WnAm) oracle: n-bit weight RTN, m-bit
activation quantizer, and the m-plane AND+popcount identity."""
import numpy as np
import pytest

from oracle import act as oact, bitserial, gemv as og, weights as ow


def _gauss(seed, shape, sigma):
    return np.random.default_rng(seed).normal(0.0, sigma, shape).astype(np.float32)


def test_wnam_two_bits_is_w2a8():
    W = _gauss(3, (16, 512), 0.02)
    a, b = ow.quantize_w2a8(W), ow.quantize_wnam(W, 2)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint16), b[1].view(np.uint16))
    assert np.array_equal(a[2].view(np.uint16), b[2].view(np.uint16))


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_wnam_rtn_invariants(n):
    L = (1 << n) - 1
    W = _gauss(10 + n, (32, 512), 0.02)
    q, delta, zero = ow.quantize_wnam(W, n)
    assert q.max() <= L
    assert np.all(np.isin(zero.astype(np.float64), np.arange(L + 1)))
    d = np.repeat(delta.astype(np.float64), 128, axis=1)
    z = np.repeat(zero.astype(np.float64), 128, axis=1)
    err = np.abs(W - d * (q - z))
    r = np.rint(W / d) + z
    unclamped = (r >= 0) & (r <= L)
    assert np.all(err[unclamped] <= d[unclamped] / 2 * (1 + 1e-9))
    assert np.all(err <= d * 1.0 + 1e-12)       # the extremes are within one step


def test_wnam_hand_cases():
    g = np.zeros(128, dtype=np.float32)
    g[0], g[1] = -0.7, 0.7
    q, delta, zero = ow.quantize_wnam(g[None, :], 3)
    # delta = fl16(1.4 / 7) = 0.199951171875; z = rint(0.7 / delta) = rint(3.5009) = 4;
    # -0.7 -> rint(-3.5009) + 4 = 0; 0.7 -> 8, clamped to 7; 0 -> 4
    assert float(delta[0, 0]) == 0.199951171875 and float(zero[0, 0]) == 4.0
    assert (q[0, 0], q[0, 1], q[0, 2]) == (0, 7, 4)
    g = np.full(128, 0.4, dtype=np.float32)
    g[0], g[1] = -0.2, 0.6
    q, delta, zero = ow.quantize_wnam(g[None, :], 1)
    # one bit: delta = fl16(0.8) = 0.7998046875, z = rint(0.25) = 0,
    # -0.2 -> 0, 0.6 -> rint(0.750) = 1, 0.4 -> rint(0.5001) = 1
    assert float(delta[0, 0]) == 0.7998046875 and float(zero[0, 0]) == 0.0
    assert (q[0, 0], q[0, 1], q[0, 2]) == (0, 1, 1)


def test_act_quant_bits_hand_cases():
    x = np.array([[7.0, -7.0, 3.5, 2.5, 0.49, -3.5] + [0.0] * 26], dtype=np.float32)
    q, d = oact.quantize(x, 4)                  # Qm = 7, s = 1
    assert list(q[0, :6]) == [7, -7, 4, 2, 0, -4] and d[0] == 1.0
    x = np.array([[1.0, -1.0, 0.5, 0.49, -0.6] + [0.0] * 27], dtype=np.float32)
    q, d = oact.quantize(x, 2)                  # Qm = 1: ternary activations
    assert list(q[0, :5]) == [1, -1, 0, 0, -1] and d[0] == 1.0
    x = _gauss(4, (3, 256), 1.0)
    assert all(np.array_equal(a, b) for a, b in zip(oact.quantize(x), oact.quantize(x, 8)))
    for m in range(2, 9):
        q, d = oact.quantize(x, m)
        Q = (1 << (m - 1)) - 1
        assert np.abs(q).max() == Q             # the absmax element maps to +-Q
        assert np.all(np.abs(q.astype(np.float64) * d[:, None] - x) <= d[:, None] / 2 * (1 + 1e-6))


@pytest.mark.parametrize("m", range(2, 9))
def test_m_bit_planes_exhaustive(m):
    Q = (1 << (m - 1)) - 1
    q = np.arange(-Q, Q + 1, dtype=np.int64)
    planes = bitserial.act_planes(q).astype(np.int64)          # [8, values]
    assert np.array_equal(bitserial.act_plane_weights(m) @ planes, q)
    if m == 8:
        assert np.array_equal(bitserial.act_plane_weights(8), bitserial.ACT_PLANE_WEIGHTS)


@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("m", [2, 3, 4, 6, 8])
def test_wnam_single_element_tables(n, m):
    """Every (n-bit code, m-bit activation) pair through the planes equals the
    integer product, at a few bit positions of a word."""
    Q = (1 << (m - 1)) - 1
    qx = np.arange(-Q, Q + 1, dtype=np.int64)
    codes = np.arange(1 << n)
    for pos in (0, 17, 31):
        xbits = np.zeros((len(qx), 32), dtype=np.int64)
        xbits[:, pos] = qx
        wbits = np.zeros((len(codes), 32), dtype=np.int64)
        wbits[:, pos] = codes
        x_words = bitserial.pack_bits(bitserial.act_planes(xbits))            # [8, X, 1]
        w_words = bitserial.pack_bits(bitserial.unsigned_planes(wbits, n))   # [n, C, 1]
        t = bitserial.and_popcount_dot(w_words, [1 << i for i in range(n)], x_words,
                                       bitserial.act_plane_weights(m))
        assert np.array_equal(t, np.outer(qx, codes))


@pytest.mark.parametrize("n,m", [(1, 8), (3, 4), (4, 4), (4, 2)])
def test_wnam_group_partials_bruteforce(n, m):
    rng = np.random.default_rng(100 * n + m)
    M, N, K = 2, 5, 256
    W = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    qw, delta, zero = ow.quantize_wnam(W, n)
    q, d = oact.quantize(rng.normal(0, 1, (M, K)).astype(np.float32), m)
    A_planes = bitserial.and_popcount_dot(bitserial.pack_bits(bitserial.unsigned_planes(qw, n)),
                                          [1 << i for i in range(n)],
                                          bitserial.pack_bits(bitserial.act_planes(q)),
                                          bitserial.act_plane_weights(m), group_words=4)
    assert np.array_equal(A_planes, og.w2a8_int(qw, q))
    # and the epilogue rebuilds the dequantized product
    S = oact.group_sums(q, 128)
    y = og.w2a8_from_int(og.w2a8_int(qw, q), S, delta, zero, d)
    y_ref, tol = og.gemv_w2a8(qw, delta, zero, q, d)
    assert np.all(np.abs(y - y_ref) <= 1e-9 * tol + 1e-12)
