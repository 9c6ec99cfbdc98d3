"""Pins of the [ABQ] §3.3 bit-balance quantizer (symmetric five-level 2-bit
grid {-2,-1,0,1,2}): hand case, mirror symmetry, levels, rounding bound,
the group maximum on the outer level, and the zero-mean property that the
asymmetric four-level grid lacks."""
import numpy as np

from oracle import gemv as og, weights as ow


def _deq(code, delta, zero):
    return og.deq_w2a8(code, delta, zero)


def test_hand_case():
    W = np.zeros((1, 128), np.float32)
    W[0, :5] = [1.0, -0.5, 0.26, -0.74, 0.76]
    code, delta, zero = ow.quantize_bit_balance(W)
    assert delta[0, 0] == np.float16(0.5) and zero[0, 0] == 2
    # W / delta = 2, -1, 0.52, -1.48, 1.52 -> t = 2, -1, 1, -1, 2
    assert list(code[0, :5]) == [4, 1, 3, 1, 4]
    assert np.all(code[0, 5:] == 2)
    np.testing.assert_array_equal(_deq(code, delta, zero)[0, :5], [1.0, -0.5, 0.5, -0.5, 1.0])


def test_mirror_symmetry():
    W = (np.random.default_rng(1).standard_normal((6, 512)) * 0.02).astype(np.float32)
    c, d, z = ow.quantize_bit_balance(W)
    c2, d2, z2 = ow.quantize_bit_balance(-W)
    np.testing.assert_array_equal(d, d2)
    np.testing.assert_array_equal(c2.astype(int), 4 - c.astype(int))
    np.testing.assert_array_equal(_deq(c2, d2, z2), -_deq(c, d, z))


def test_levels_rounding_and_outer_level():
    W = (np.random.default_rng(2).standard_normal((16, 1024)) * 0.02).astype(np.float32)
    c, d, z = ow.quantize_bit_balance(W)
    assert c.max() <= 4 and set(np.unique(c)) == {0, 1, 2, 3, 4}
    Wh = _deq(c, d, z)
    step = np.repeat(d.astype(np.float64), 128, axis=1)
    t = Wh / step
    np.testing.assert_array_equal(t, np.rint(t))
    assert np.all(np.abs(t) <= 2)
    # round to nearest: within half a step wherever the grid reaches
    inside = np.abs(W) <= 2.5 * step
    assert inside.all()
    assert np.all(np.abs(W - Wh) <= 0.5 * step + 1e-12)
    # the largest |W| of every group lands on an outer level (+-2)
    g = np.abs(W.reshape(16, 8, 128)).argmax(-1)
    tg = t.reshape(16, 8, 128)
    outer = np.take_along_axis(tg, g[..., None], -1)[..., 0]
    assert np.all(np.abs(outer) == 2)


def test_symmetric_group_keeps_zero_mean_where_int2_does_not():
    rng = np.random.default_rng(3)
    half = (rng.standard_normal((4, 64)) * 0.02).astype(np.float32)
    W = np.concatenate([half, -half], axis=1)            # each group is symmetric
    c, d, z = ow.quantize_bit_balance(W)
    assert np.all(_deq(c, d, z).sum(axis=1) == 0.0)
    qa, da, za = ow.quantize_w2a8(W)                      # the asymmetric 4-level grid
    assert np.any(np.abs(_deq(qa, da, za).sum(axis=1)) > 0.0)


def test_degenerate_group():
    W = np.zeros((2, 256), np.float32)
    W[1, 128:] = 0.3
    c, d, z = ow.quantize_bit_balance(W)
    assert d[0, 0] == 1 and np.all(c[0] == 2) and np.all(c[1, :128] == 2)
    assert np.all(_deq(c, d, z)[0] == 0)
