"""Pins of the RaBiT iterative residual SVID (Gauss-Seidel refinement of the
paths) in the oracle."""
import numpy as np
import pytest

from oracle import weights as ow


def _gauss(seed, shape, sigma=0.02):
    return np.random.default_rng(seed).normal(0.0, sigma, shape).astype(np.float32)


def _err(W, B, g, h):
    What = sum(ow.rabit_path(B[p], g[p], h[p]) for p in range(B.shape[0]))
    return float(np.sum((W.astype(np.float64) - What) ** 2))


def test_zero_sweeps_is_the_greedy_pass():
    W = _gauss(1, (48, 256))
    a, b = ow.quantize_rabit(W, 2), ow.quantize_rabit(W, 2, svid_sweeps=0)
    assert all(np.array_equal(x.view(np.uint8), y.view(np.uint8)) for x, y in zip(a, b))


@pytest.mark.parametrize("P", [2, 3])
def test_sweeps_do_not_increase_the_error_and_beat_greedy(P):
    W = _gauss(2 + P, (64, 320))
    B, g, h = ow.quantize_rabit(W, P)
    errs = [_err(W, B, g, h)]
    for _ in range(20):
        ow.refine_rabit_svid(W, B, g, h, sweeps=1)
        errs.append(_err(W, B, g, h))
    for e0, e1 in zip(errs, errs[1:]):
        assert e1 <= e0 * (1 + 1e-6)                 # fp16 scale rounding only
    assert errs[-1] < errs[0] * 0.995                # a real improvement on Gaussian weights
    assert np.all(g.astype(np.float64) >= 0) and np.all(h.astype(np.float64) >= 0)


def test_last_path_is_the_sign_of_what_the_others_leave():
    W = _gauss(7, (40, 256))
    B, g, h = ow.quantize_rabit(W, 2, svid_sweeps=3)
    T = W.astype(np.float64) - ow.rabit_path(B[0], g[0], h[0])
    assert np.array_equal(B[1], np.where(T >= 0, 1, -1).astype(np.int8))


def test_one_path_sweep_is_idempotent():
    # one path: the target is W itself, so every sweep recomputes the greedy
    # path exactly
    W = _gauss(8, (32, 128))
    a = ow.quantize_rabit(W, 1)
    b = ow.quantize_rabit(W, 1, svid_sweeps=4)
    assert all(np.array_equal(x.view(np.uint8), y.view(np.uint8)) for x, y in zip(a, b))
