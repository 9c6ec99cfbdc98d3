"""Pins of the oracle's weight quantizers (oracle/weights.py) against
closed forms, library routines (SVD, quantile), brute force and hand cases."""
import math

import numpy as np
import pytest

from oracle import weights as ow
from oracle.common import sign_pm1


def _gauss(seed, shape, sigma):
    return (np.random.default_rng(seed).standard_normal(shape) * sigma).astype(np.float32)


# ------------------------------------------------------------------- sign
def test_sign_quantizer():
    W = _gauss(1, (16, 64), 1.0)
    W[0, 0] = 0.0
    B, alpha = ow.quantize_sign(W)
    assert B[0, 0] == 1
    assert set(np.unique(B)) <= {-1, 1}
    for n in range(16):
        assert alpha[n] == np.float32(sum(abs(float(v)) for v in W[n]) / 64)


# ------------------------------------------------------------ rank-1 / RaBiT
def test_rank1_fit_matches_svd():
    A = np.abs(_gauss(2, (64, 48), 1.0)).astype(np.float64)
    u, v, sigma = ow.rank1_fit(A, iters=200)
    U, s, Vt = np.linalg.svd(A)
    assert abs(sigma - s[0]) / s[0] <= 1e-10
    assert np.all(u >= 0) and np.all(v >= 0)
    assert np.allclose(np.abs(U[:, 0]), u, atol=1e-8)
    assert np.allclose(np.abs(Vt[0]), v, atol=1e-8)


def test_rank1_fit_converges_at_30_iterations_on_workload_shapes():
    A = np.abs(_gauss(3, (512, 256), 0.02)).astype(np.float64)
    u, v, sigma = ow.rank1_fit(A, iters=30)
    assert np.linalg.norm(A @ v - sigma * u) / sigma <= 1e-8


def test_rank1_fit_exact_on_rank1_input():
    a = np.linspace(0.5, 2.0, 32)
    b = np.linspace(0.1, 1.0, 48)
    g, h = ow.rabit_scales(np.outer(a, b))
    rec = g.astype(np.float64)[:, None] * h.astype(np.float64)[None, :]
    assert np.allclose(rec, np.outer(a, b), rtol=2e-3)


def test_rank1_zero_matrix():
    g, h = ow.rabit_scales(np.zeros((4, 8)))
    assert np.all(g == 0) and np.all(h == 0)


def test_rabit_residual_recursion_invariant():
    # [RaBiT] §2.2: B1 = sign(W), R1 = W - g1.B1.h1, B2 = sign(R1)
    W = _gauss(4, (96, 160), 0.02)
    B, g, h = ow.quantize_rabit(W, paths=2)
    assert np.array_equal(B[0], sign_pm1(W))
    R1 = W.astype(np.float64) - (g[0].astype(np.float64)[:, None] * B[0]) \
        * h[0].astype(np.float64)[None, :]
    assert np.array_equal(B[1], sign_pm1(R1))
    assert np.all(g >= 0) and np.all(h >= 0)
    # the second path reduces the reconstruction error
    W1 = (g[0].astype(np.float64)[:, None] * B[0]) * h[0].astype(np.float64)[None, :]
    W2 = W1 + (g[1].astype(np.float64)[:, None] * B[1]) * h[1].astype(np.float64)[None, :]
    e1 = np.mean((W - W1) ** 2)
    e2 = np.mean((W - W2) ** 2)
    assert e2 < e1
    # one path with the optimal scales beats a per-row alpha (sign format)
    Bs, alpha = ow.quantize_sign(W)
    es = np.mean((W - alpha.astype(np.float64)[:, None] * Bs) ** 2)
    assert e1 <= es * 1.0001


def test_rabit_one_path_unit_scales_is_sign():
    from oracle import gemv
    W = _gauss(5, (8, 64), 1.0)
    B = sign_pm1(W)[None]
    g = np.ones((1, 8), np.float16)
    h = np.ones((1, 64), np.float16)
    assert np.array_equal(gemv.deq_rabit(B, g, h), B[0].astype(np.float64))


# ------------------------------------------------------------------ ternary
def test_ternary_identity_and_hand_case():
    W = np.array([[0.1, -0.1, 0.01, 0.3, -0.3, 0.049]], dtype=np.float32)
    T, gamma = ow.quantize_ternary(W)
    # gamma = mean |W| = 0.859/6
    assert gamma == np.float32(np.mean(np.abs(W.astype(np.float64))))
    # W/gamma = 0.698, -0.698, 0.0698, 2.095, -2.095, 0.342
    assert T.tolist() == [[1, -1, 0, 1, -1, 0]]
    # [HGF] §1.2: w.x in {-x, 0, x}
    x = np.float32(1.75)
    for t in T[0]:
        assert t * x in (-x, 0, x)


def test_ternary_zero_fraction_gaussian():
    # T = 0 iff |W| < gamma/2 and gamma = E|W| = sigma sqrt(2/pi), so
    # P(T = 0) = erf(0.5 sqrt(2/pi) / sqrt 2) = 0.3101 for Gaussian W.
    W = _gauss(6, (512, 512), 0.02)
    T, _ = ow.quantize_ternary(W)
    frac = np.mean(T == 0)
    expect = math.erf(0.5 * math.sqrt(2 / math.pi) / math.sqrt(2))
    assert abs(expect - 0.3101) < 1e-4
    assert abs(frac - expect) < 0.005


# --------------------------------------------------------------------- W2A8
def test_w2a8_hand_case():
    g = np.zeros(128, dtype=np.float32)
    g[0], g[1], g[2] = -0.3, 0.3, 0.0
    q, delta, zero = ow.quantize_w2a8(g[None, :])
    # delta = fl16(0.6/3) = 0.199951171875; z = rint(0.3/delta) = rint(1.5004) = 2
    assert float(delta[0, 0]) == 0.199951171875
    assert float(zero[0, 0]) == 2.0
    assert q[0, 0] == 0 and q[0, 1] == 3 and q[0, 2] == 2


def test_w2a8_rtn_invariants():
    W = _gauss(7, (32, 512), 0.02)
    q, delta, zero = ow.quantize_w2a8(W)
    assert q.max() <= 3
    assert np.all(np.isin(zero.astype(np.float64), [0, 1, 2, 3]))
    d = np.repeat(delta.astype(np.float64), 128, axis=1)
    z = np.repeat(zero.astype(np.float64), 128, axis=1)
    What = d * (q - z)
    err = np.abs(W - What)
    unclamped = (np.rint(W / d) + z >= 0) & (np.rint(W / d) + z <= 3)
    assert np.all(err[unclamped] <= d[unclamped] / 2 * (1 + 1e-9))
    # the group extremes lie within one step of the grid ends
    assert np.all(err <= d * 1.0 + 1e-12)


def test_w2a8_degenerate_group():
    W = np.full((1, 256), 0.01, dtype=np.float32)
    W[0, 128:] = _gauss(8, 128, 0.02)
    q, delta, zero = ow.quantize_w2a8(W)
    assert float(delta[0, 0]) == 1.0 and float(zero[0, 0]) == 0.0
    assert np.all(q[0, :128] == 0)


# --------------------------------------------------------------------- BVSR
def test_bvsr_cache_structure():
    W = _gauss(9, (64, 512), 0.015)
    cache = ow.bvsr_cache(W)
    Wg = W.reshape(-1, 32).astype(np.float64)
    spans = Wg.max(1) - Wg.min(1)
    for i in range(16):
        r = 1.6 + 0.8 * i / 15
        for j in range(16):
            c = cache[16 * i + j].astype(np.float64)
            L = np.quantile(spans, (j + 0.5) / 16)          # library routine
            assert abs(c[:4].sum() - L) <= 1e-6 * L
            assert abs(c[4] + L / 2) <= 1e-6 * L
            assert np.allclose(c[1:4] / c[0:3], r, rtol=1e-6)
    L = np.array([-2 * cache[j, 4] for j in range(16)])
    assert np.all(np.diff(L) >= 0)


def test_bvsr_ratio_two_is_uniform_grid():
    # with r = 2 the 16 subset sums are b + a*{0..15}: the plain 4-bit grid
    a, b = np.float32(0.01), np.float32(-0.075)
    cache = np.zeros((1, 5), np.float32)
    cache[0] = (a, 2 * a, 4 * a, 8 * a, b)
    pts = ow.bvsr_points(cache)[0]
    assert np.array_equal(pts, np.float64(b) + np.float64(a) * np.arange(16))


def test_bvsr_encode_nearest_bruteforce_and_ties():
    W = _gauss(10, (4, 64), 0.015)
    cache = ow.bvsr_cache(W)
    idx = np.array([[3, 200], [17, 255], [0, 128], [77, 99]], dtype=np.uint8)
    code, sse = ow.bvsr_encode(W, cache, idx)
    pts = ow.bvsr_points(cache)
    for n in range(4):
        for g in range(2):
            p = pts[idx[n, g]]
            s = 0.0
            for e in range(32):
                w = float(W[n, 32 * g + e])
                dists = [(w - p[c]) ** 2 for c in range(16)]
                best = min(range(16), key=lambda c: (dists[c], c))
                assert code[n, 32 * g + e] == best
                s += dists[best]
            assert abs(s - sse[n, g]) <= 1e-15 * max(s, 1e-30)
    # a weight exactly midway between two points goes to the smaller code
    cache2 = np.zeros((1, 5), np.float32)
    cache2[0] = (1.0, 2.0, 4.0, 8.0, 0.0)
    Wt = np.zeros((1, 32), np.float32)
    Wt[0, 0] = 2.5
    code2, _ = ow.bvsr_encode(Wt, cache2, np.zeros((1, 1), np.uint8))
    assert code2[0, 0] == 2


def test_bvsr_search_is_argmin_over_all_sets():
    W = _gauss(11, (6, 128), 0.015)
    cache = ow.bvsr_cache(W)
    code, idx, sse = ow.bvsr_search(W, cache)
    all_sse = np.stack([ow.bvsr_encode(W, cache, np.full((6, 4), s, np.uint8))[1]
                        for s in range(256)])                      # [256, 6, 4]
    assert np.array_equal(sse, all_sse.min(axis=0))
    assert np.array_equal(idx, np.argmin(all_sse, axis=0))          # first = lowest id
    c2, _ = ow.bvsr_encode(W, cache, idx)
    assert np.array_equal(code, c2)
    # BVSR beats the best single uniform grid on the same data (sanity)
    assert sse.mean() < all_sse.mean(axis=(1, 2)).min() * 1.0 + 1e-30
