"""Pins of the fully binary (XNOR+popcount) oracle: activation binarizer,
packed sign words, the exact integer product and its float form."""
import numpy as np

from oracle import act as oact, bitserial, gemv as og, weights as ow


def test_binarize_hand_cases():
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :6] = [0.0, -0.0, 1e-30, -1e-30, 2.0, -3.0]
    xb, beta = oact.binarize(x)
    assert list(xb[0, :6]) == [1, 1, 1, -1, 1, -1]          # sign(0) = +1, also for -0.0
    assert np.all(xb[0, 6:] == 1)
    assert beta[0] == (2.0 + 3.0 + 2e-30) / 32


def test_binary_words_positions_and_padding():
    xb = np.full((2, 64), -1, dtype=np.int8)
    xb[0, 0] = xb[0, 33] = xb[1, 63] = 1
    w = oact.binary_words(xb, Kp=128)
    assert w.shape == (2, 4) and w.dtype == np.uint32
    assert list(w[0]) == [1, 2, 0, 0] and list(w[1]) == [0, 1 << 31, 0, 0]


def test_xnor_int_is_popcount_identity_with_padding():
    rng = np.random.default_rng(5)
    N, K, Kp = 7, 96, 128
    B = rng.choice([-1, 1], size=(N, K)).astype(np.int8)
    xb = rng.choice([-1, 1], size=(3, K)).astype(np.int8)
    bits = np.zeros((N, Kp), dtype=np.uint8)
    bits[:, :K] = B > 0
    bw = bitserial.pack_bits(bits)
    xw = oact.binary_words(xb, Kp)
    for m in range(3):
        # zero padding bits on both sides agree, so XOR counts only real mismatches
        assert np.array_equal(bitserial.xnor_popcount_dot(bw, xw[m], K), og.xnor_int(B, xb)[m])


def test_xnor_gemv_reduces_to_sign_gemv_for_constant_magnitude():
    rng = np.random.default_rng(6)
    N, K = 40, 256
    B, alpha = ow.quantize_sign(rng.normal(0, 1, (N, K)).astype(np.float32))
    s = rng.choice([-1.0, 1.0], size=(2, K)).astype(np.float32)
    x = (s * np.float32(0.75)).astype(np.float32)               # |x| constant: beta * x_b = x
    xb, beta = oact.binarize(x)
    y1, _ = og.gemv_xnor(B, alpha, xb, beta)
    y2, _ = og.gemv_sign(B, alpha, x)
    assert np.allclose(y1, y2, rtol=1e-12, atol=0)
    # and it is alpha * beta * (integer product), row by row
    Y = og.xnor_int(B, xb)
    for m in range(2):
        for n in (0, 17, N - 1):
            assert abs(y1[m, n] - float(alpha[n]) * beta[m] * Y[m, n]) <= 1e-12 * abs(y1[m, n]) + 1e-15
