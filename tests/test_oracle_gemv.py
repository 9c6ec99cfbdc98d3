"""Pins of oracle/gemv.py: fp64 GEMV vs explicit loops, int64 partials vs the
explicit dequantized product, the factorized forms the kernels evaluate, and
batch invariance."""
import numpy as np

from oracle import act, gemv, weights as ow
import synth


def _loop_gemv(What, xhat):
    M, K = xhat.shape
    N = What.shape[0]
    y = np.zeros((M, N))
    b = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            s = 0.0
            a = 0.0
            for k in range(K):
                s += float(What[n, k]) * float(xhat[m, k])
                a += abs(float(What[n, k]) * float(xhat[m, k]))
            y[m, n], b[m, n] = s, a
    return y, 2e-3 * b


def test_sign_gemv_vs_loop_and_all_plus_row():
    W = synth.gaussian_f32(np.random.default_rng(0), (6, 64), 1.0)
    W[2] = np.abs(W[2])                       # all +1 row
    x = synth.gaussian_f32(np.random.default_rng(1), (1, 64), 1.0)
    B, alpha = ow.quantize_sign(W)
    y, tol = gemv.gemv_sign(B, alpha, x)
    yl, tl = _loop_gemv(alpha.astype(np.float64)[:, None] * B, x)
    assert np.allclose(y, yl, rtol=1e-13, atol=1e-13) and np.allclose(tol, tl, rtol=1e-12)
    assert abs(y[0, 2] - float(alpha[2]) * x[0].astype(np.float64).sum()) < 1e-12


def test_rabit_gemv_and_factorization():
    W = synth.gaussian_f32(np.random.default_rng(2), (40, 96), 0.02)
    _, x = synth.random_bf16(np.random.default_rng(3), (1, 96))
    B, g, h = ow.quantize_rabit(W)
    y, tol = gemv.gemv_rabit(B, g, h, x)
    yl, tl = _loop_gemv(gemv.deq_rabit(B, g, h), x)
    assert np.allclose(y, yl, rtol=1e-12, atol=1e-15) and np.allclose(tol, tl, rtol=1e-12)
    # the form the sign-apply kernel evaluates: sum_p g_p (B_p (h_p x))
    xf = x[0].astype(np.float64)
    yf = sum(g[p].astype(np.float64) * (B[p].astype(np.float64) @ (h[p].astype(np.float64) * xf))
             for p in range(2))
    assert np.allclose(yf, y[0], rtol=1e-12, atol=1e-15)


def test_ternary_int_and_epilogue():
    W = synth.gaussian_f32(np.random.default_rng(4), (24, 128), 0.02)
    _, x = synth.random_bf16(np.random.default_rng(5), (3, 128))
    T, gamma = ow.quantize_ternary(W)
    q, d = act.quantize(x)
    Y = gemv.ternary_int(T, q)
    for m in range(3):
        for n in range(24):
            assert Y[m, n] == sum(int(T[n, k]) * int(q[m, k]) for k in range(128))
    y, tol = gemv.gemv_ternary(T, gamma, q, d)
    assert np.allclose(gemv.ternary_from_int(Y, gamma, d), y, rtol=1e-12, atol=1e-15)
    yl, _ = _loop_gemv(float(gamma) * T.astype(np.float64), gemv.act_hat(q, d))
    assert np.allclose(y, yl, rtol=1e-12, atol=1e-15)


def test_w2a8_int_zero_point_identity():
    W = synth.gaussian_f32(np.random.default_rng(6), (16, 256), 0.02)
    _, x = synth.random_bf16(np.random.default_rng(7), (2, 256))
    x[:, 5] *= 20
    qw, delta, zero = ow.quantize_w2a8(W)
    q, d = act.quantize(x)
    A = gemv.w2a8_int(qw, q)
    S = act.group_sums(q, 128)
    for m in range(2):
        for n in range(16):
            for g in range(2):
                assert A[m, n, g] == sum(int(qw[n, k]) * int(q[m, k])
                                         for k in range(128 * g, 128 * g + 128))
    y, tol = gemv.gemv_w2a8(qw, delta, zero, q, d)
    # sum delta (q - z) x = delta (sum q x - z sum x)
    assert np.allclose(gemv.w2a8_from_int(A, S, delta, zero, d), y, rtol=1e-12, atol=1e-15)
    # a group whose codes all equal the zero point contributes nothing
    qw2 = qw.copy()
    qw2[3, :128] = int(zero[3, 0])
    A2 = gemv.w2a8_int(qw2, q)
    t = float(delta[3, 0]) * (A2[:, 3, 0] - float(zero[3, 0]) * S[:, 0])
    assert np.all(t == 0)


def test_bvsr_int_and_epilogue():
    W = synth.gaussian_f32(np.random.default_rng(8), (8, 128), 0.015)
    _, x = synth.random_bf16(np.random.default_rng(9), (2, 128))
    cache = ow.bvsr_cache(W)
    code, idx, _ = ow.bvsr_search(W, cache)
    q, d = act.quantize(x)
    P = gemv.bvsr_int(code, q)
    for m in range(2):
        for n in range(8):
            for g in range(4):
                for b in range(4):
                    assert P[m, n, g, b] == sum(((int(code[n, k]) >> b) & 1) * int(q[m, k])
                                                for k in range(32 * g, 32 * g + 32))
    S = act.group_sums(q, 32)
    y, tol = gemv.gemv_bvsr(code, idx, cache, q, d)
    assert np.allclose(gemv.bvsr_from_int(P, S, idx, cache, d), y, rtol=1e-12, atol=1e-15)
    # r = 2 closed form: sum_b 2^b P_b = sum_k code_k q_k
    tot = (P * np.array([1, 2, 4, 8])).sum(-1).sum(-1)
    assert np.array_equal(tot, q.astype(np.int64) @ code.astype(np.int64).T)


def test_batch_invariance_of_act_quant_and_int_gemv():
    W = synth.gaussian_f32(np.random.default_rng(10), (12, 256), 0.02)
    _, x = synth.random_bf16(np.random.default_rng(11), (16, 256))
    qw, delta, zero = ow.quantize_w2a8(W)
    q, d = act.quantize(x)
    A = gemv.w2a8_int(qw, q)
    for m in [0, 7, 15]:
        q1, d1 = act.quantize(x[m:m + 1])
        assert np.array_equal(q1[0], q[m]) and d1[0] == d[m]
        assert np.array_equal(gemv.w2a8_int(qw, q1)[0], A[m])


def test_tolerance_is_relative_to_abs_products():
    What = np.array([[1.0, -1.0], [2.0, 0.0]])
    xhat = np.array([[3.0, 3.0]])
    y, tol = gemv._chunked_matmul(lambda a, b: What[a:b], 2, xhat)
    assert y.tolist() == [[0.0, 6.0]]
    assert np.allclose(tol, [[2e-3 * 6.0, 2e-3 * 6.0]])
