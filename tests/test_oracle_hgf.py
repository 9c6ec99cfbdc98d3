"""Pins of the HGF oracle ([HGF] §2.1 gated low-rank correction, §4.1 fused
ternary + correction layer): SiLU special values and identities, a hand case
whose result is a closed form, the zero-initialized correction, and brute
force on tiny inputs."""
import math

import numpy as np

from oracle import gemv as og

LN3 = math.log(3.0)


def test_silu_special_values():
    # sigmoid(ln a) = a / (1 + a), so silu(ln 3) = 0.75 ln 3, silu(-ln 3) = -0.25 ln 3
    got = og.silu(np.array([0.0, LN3, -LN3, math.log(9.0)]))
    want = [0.0, 0.75 * LN3, -0.25 * LN3, 0.9 * math.log(9.0)]
    np.testing.assert_allclose(got, want, rtol=1e-15, atol=0)


def test_silu_odd_part_identity():
    # silu(z) - silu(-z) = z (sigmoid(z) + sigmoid(-z) = 1)
    z = np.random.default_rng(3).normal(0, 4, 1000)
    np.testing.assert_allclose(og.silu(z) - og.silu(-z), z, rtol=0, atol=1e-13)


def test_silu_minimum_and_limits():
    # at the minimum x*, silu'(x*) = 0 gives sigmoid = (x* + 1) / x*, so
    # silu(x*) = x* + 1 (x* ~ -1.2785)
    z = np.linspace(-3.0, 0.0, 300001)       # step 1e-5
    v = og.silu(z)
    i = int(np.argmin(v))
    # z + 1 has slope 1 where silu is flat: the grid point is off by < 1e-5
    assert abs(v[i] - (z[i] + 1.0)) < 1e-5
    assert abs(v[i] + 0.2784645) < 1e-6
    assert -1.30 < z[i] < -1.25
    assert og.silu(np.array([40.0]))[0] == np.float64(40.0) or \
        abs(og.silu(np.array([40.0]))[0] / 40.0 - 1) < 1e-15
    with np.errstate(all="raise"):
        assert og.silu(np.array([-800.0]))[0] == 0.0     # -0.0, no overflow warning


def test_gate_is_tanh_and_bounded():
    # tanh(ln 2) = (2 - 1/2) / (2 + 1/2) = 0.6
    assert abs(og.lora_gate(math.log(2.0)) - 0.6) < 1e-15
    assert og.lora_gate(0.0) == 0.0
    for a in (-30.0, -3.0, 0.1, 3.0, 30.0):
        assert abs(og.lora_gate(a)) <= 1.0
    assert og.lora_gate(-0.5) == -og.lora_gate(0.5)


def _hand_case():
    """K = 3, r = 2, N = 3, two tokens; z = x A = (ln 3, -ln 3) for token 0
    and 0 for token 1; gate tanh(ln 2) = 0.6."""
    x = np.array([[1.0, 2.0, -1.0], [0.0, 0.0, 0.0]])
    A = np.array([[LN3, 0.0], [0.5 * LN3, -0.5 * LN3], [LN3, 0.0]])      # [K, r]
    B = np.array([[4.0, -8.0, 1.0], [4.0, 12.0, 2.0]])                    # [r, N]
    return x, A, B, math.log(2.0)


def test_lora_correction_hand_case():
    x, A, B, alpha = _hand_case()
    out, tol = og.lora_correction(x, A, B, alpha)
    # h = (0.75 L, -0.25 L): h B = (2 L, -9 L, 0.25 L); times 0.6
    want = np.array([[1.2 * LN3, -5.4 * LN3, 0.15 * LN3], [0.0, 0.0, 0.0]])
    np.testing.assert_allclose(out, want, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(og.lora_down(x, A), [[0.75 * LN3, -0.25 * LN3], [0.0, 0.0]],
                               rtol=1e-14, atol=1e-15)
    assert np.all(tol >= og.TOL_REL * np.abs(out) - 1e-18)


def test_gemv_hgf_hand_case():
    x, A, B, alpha = _hand_case()
    T = np.array([[1, 0, -1], [-1, 1, 0], [0, 0, 1]], dtype=np.int8)
    q = np.array([[10, -20, 30], [0, 0, 0]], dtype=np.int8)
    d = np.array([0.1, 0.0], dtype=np.float32)
    y, _ = og.gemv_hgf(T, np.float32(0.5), q, d, x, A, B, alpha)
    # ternary: Y = (-20, -30, 30), gamma d = 0.05 (d is fp32 0.1)
    gd = 0.5 * float(np.float32(0.1))
    want0 = np.array([-20 * gd + 1.2 * LN3, -30 * gd - 5.4 * LN3, 30 * gd + 0.15 * LN3])
    np.testing.assert_allclose(y[0], want0, rtol=1e-14)
    np.testing.assert_array_equal(y[1], [0.0, 0.0, 0.0])


def test_zero_initialized_correction_is_plain_ternary():
    # [HGF] §2.1 starts B at zero (and a zero gate also removes the path)
    rng = np.random.default_rng(11)
    N, K, r = 40, 96, 8
    T = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    q = rng.integers(-127, 128, size=(2, K)).astype(np.int8)
    d = np.array([0.02, 0.5], dtype=np.float32)
    x = rng.normal(size=(2, K))
    A = rng.normal(0, 0.02, size=(K, r))
    yt, tt = og.gemv_ternary(T, np.float32(0.03), q, d)
    y0, t0 = og.gemv_hgf(T, np.float32(0.03), q, d, x, A, np.zeros((r, N)), 0.1)
    np.testing.assert_array_equal(y0, yt)
    B = rng.normal(0, 0.02, size=(r, N))
    y1, _ = og.gemv_hgf(T, np.float32(0.03), q, d, x, A, B, 0.0)
    np.testing.assert_array_equal(y1, yt)


def test_lora_brute_force_loops():
    rng = np.random.default_rng(12)
    M, K, r, N = 2, 7, 3, 5
    x = rng.normal(size=(M, K))
    A = rng.normal(0, 0.5, size=(K, r))
    B = rng.normal(0, 0.5, size=(r, N))
    alpha = -0.7
    out, _ = og.lora_correction(x, A, B, alpha)
    gate = math.tanh(alpha)
    for m in range(M):
        h = []
        for j in range(r):
            z = 0.0
            for k in range(K):
                z += x[m, k] * A[k, j]
            h.append(z / (1.0 + math.exp(-z)))
        for n in range(N):
            s = 0.0
            for j in range(r):
                s += h[j] * B[j, n]
            assert abs(out[m, n] - gate * s) <= 1e-13 * (1 + abs(gate * s))


def test_rank_split_additivity():
    # the rank components are independent: rank r = rank r1 + rank r - r1
    rng = np.random.default_rng(13)
    K, r, N = 64, 8, 24
    x = rng.normal(size=(3, K))
    A = rng.normal(0, 0.1, size=(K, r))
    B = rng.normal(0, 0.1, size=(r, N))
    full, _ = og.lora_correction(x, A, B, 0.3)
    a, _ = og.lora_correction(x, A[:, :3], B[:3], 0.3)
    b, _ = og.lora_correction(x, A[:, 3:], B[3:], 0.3)
    np.testing.assert_allclose(full, a + b, rtol=1e-12, atol=1e-15)
