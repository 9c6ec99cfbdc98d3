"""Pins of oracle/bitserial.py and oracle/act.py against exhaustive tables,
brute force and hand-worked cases (CPU only)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import act, bitserial
from oracle.common import sign_pm1


# ------------------------------------------------------------------- sign
def test_sign_tie_rule():
    # [BitNet] §2.1: sign(x) = +1 if x >= 0 else -1; zeros (both signs) -> +1
    v = np.array([-1.0, -0.0, 0.0, 1e-30, -1e-30, 3.0], dtype=np.float32)
    assert sign_pm1(v).tolist() == [-1, 1, 1, 1, -1, 1]


# ------------------------------------------------------------- bit packing
def test_pack_bits_lsb_first_positions():
    K = 96
    for k in [0, 1, 31, 32, 33, 63, 64, 95]:
        e = np.zeros(K, dtype=np.uint8)
        e[k] = 1
        w = bitserial.pack_bits(e)
        expect = np.zeros(3, dtype=np.uint32)
        expect[k // 32] = np.uint32(1) << np.uint32(k % 32)
        assert np.array_equal(w, expect), k
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2, size=(5, 7, 128)).astype(np.uint8)
    assert np.array_equal(bitserial.unpack_bits(bitserial.pack_bits(bits)), bits)


def test_act_planes_exhaustive_twos_complement():
    # every int8 value is rebuilt from its 8 planes with weights 1..64, -128
    q = np.arange(-128, 128, dtype=np.int64).astype(np.int8)
    X = bitserial.act_planes(q).astype(np.int64)          # [8, 256]
    rebuilt = (bitserial.ACT_PLANE_WEIGHTS[:, None] * X).sum(axis=0)
    assert np.array_equal(rebuilt, q.astype(np.int64))
    # plane j is bit j of the byte: q = 1 sets only plane 0, q = -1 sets all
    assert X[:, 128 + 1].tolist() == [1, 0, 0, 0, 0, 0, 0, 0]
    assert X[:, 128 - 1].tolist() == [1] * 8


def _single_element_table(wcodes, wplanes_fn, wweights, pos):
    """Rows = each weight code at channel `pos`, tokens = each int8 value at
    `pos`, zeros elsewhere; returns the AND+popcount result [256, n_codes]."""
    K = 64
    n = len(wcodes)
    Wc = np.zeros((n, K), dtype=np.int64)
    Wc[:, pos] = wcodes
    q = np.zeros((256, K), dtype=np.int8)
    q[:, pos] = np.arange(-128, 128).astype(np.int8)
    w_words = bitserial.pack_bits(wplanes_fn(Wc))
    x_words = bitserial.pack_bits(bitserial.act_planes(q))
    return bitserial.and_popcount_dot(w_words, wweights, x_words, bitserial.ACT_PLANE_WEIGHTS)


@pytest.mark.parametrize("pos", [0, 5, 31, 32, 63])
def test_single_element_tables(pos):
    qx = np.arange(-128, 128, dtype=np.int64)
    # W2A8: 2-bit unsigned weight codes, plane weights 1, 2
    t = _single_element_table([0, 1, 2, 3], lambda c: bitserial.unsigned_planes(c, 2), [1, 2], pos)
    assert np.array_equal(t, np.outer(qx, [0, 1, 2, 3]))
    # BVSR: 4 bitvectors, plane weights 1, 2, 4, 8 (the r = 2 grid)
    t = _single_element_table(list(range(16)), lambda c: bitserial.unsigned_planes(c, 4),
                              [1, 2, 4, 8], pos)
    assert np.array_equal(t, np.outer(qx, np.arange(16)))
    # ternary as plus/minus planes with weights +1, -1 ([HGF] §1.2 identity
    # w.x in {-x, 0, x})
    t = _single_element_table([-1, 0, 1],
                              lambda c: np.stack([(c == 1), (c == -1)]).astype(np.uint8),
                              [1, -1], pos)
    assert np.array_equal(t, np.outer(qx, [-1, 0, 1]))


@settings(max_examples=40, deadline=None)
@given(st.integers(1, 4), st.integers(1, 5), st.integers(1, 4), st.integers(0, 2**31 - 1))
def test_and_popcount_equals_int_dot_bruteforce(M, N, kw, seed):
    rng = np.random.default_rng(seed)
    K = 32 * kw
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    x_words = bitserial.pack_bits(bitserial.act_planes(q))
    qi = q.astype(np.int64)
    # 2-bit weights
    qw = rng.integers(0, 4, size=(N, K))
    got = bitserial.and_popcount_dot(bitserial.pack_bits(bitserial.unsigned_planes(qw, 2)),
                                     [1, 2], x_words, bitserial.ACT_PLANE_WEIGHTS)
    ref = np.array([[sum(int(qi[m, k]) * int(qw[n, k]) for k in range(K)) for n in range(N)]
                    for m in range(M)])
    assert np.array_equal(got, ref)
    # 4-bit codes, grouped per word
    code = rng.integers(0, 16, size=(N, K))
    got = bitserial.and_popcount_dot(bitserial.pack_bits(bitserial.unsigned_planes(code, 4)),
                                     [1, 2, 4, 8], x_words, bitserial.ACT_PLANE_WEIGHTS,
                                     group_words=1)
    ref = (code.reshape(1, N, kw, 32) * qi.reshape(M, 1, kw, 32)).sum(-1)
    assert np.array_equal(got, ref)
    # ternary
    T = rng.integers(-1, 2, size=(N, K))
    planes = np.stack([(T == 1), (T == -1)]).astype(np.uint8)
    got = bitserial.and_popcount_dot(bitserial.pack_bits(planes), [1, -1], x_words,
                                     bitserial.ACT_PLANE_WEIGHTS)
    assert np.array_equal(got, qi @ T.T)


def test_xnor_popcount_identity():
    # [BitNet] §2.3 XNOR+popcount: for +-1 vectors, a.b = K - 2 popcount(a^b)
    rng = np.random.default_rng(3)
    K = 256
    B = rng.choice([-1, 1], size=(8, K))
    s = rng.choice([-1, 1], size=K)
    bw = bitserial.pack_bits((B > 0).astype(np.uint8))
    sw = bitserial.pack_bits((s > 0).astype(np.uint8))
    assert np.array_equal(bitserial.xnor_popcount_dot(bw, sw, K), B @ s)


# ------------------------------------------------------ activation quantizer
def test_act_quant_hand_cases():
    # all zero -> q = 0, d = 0
    q, d = act.quantize(np.zeros((1, 4), dtype=np.float32))
    assert q.tolist() == [[0, 0, 0, 0]] and d.tolist() == [0.0]
    # amax = 2: s = 63.5, 1.0 * 63.5 = 63.5 is an exact tie -> 64 (half even)
    q, d = act.quantize(np.array([[2.0, -2.0, 1.0, -1.0, 0.0]], dtype=np.float32))
    assert q.tolist() == [[127, -127, 64, -64, 0]]
    assert d[0] == np.float32(2.0) / np.float32(127.0)
    # amax = 127: s = 1 exactly, ties round to even
    x = np.array([[127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5]], dtype=np.float32)
    q, d = act.quantize(x)
    assert q.tolist() == [[127, 2, 4, -2, -4, 0, 2]]
    assert d[0] == np.float32(1.0)


@settings(max_examples=200, deadline=None)
@given(st.floats(min_value=1e-30, max_value=1e30, allow_nan=False, allow_infinity=False),
       st.integers(0, 2**31 - 1))
def test_act_quant_properties(scale, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((2, 96)) * scale).astype(np.float32)
    if not np.all(np.isfinite(x)) or np.max(np.abs(x)) == 0:
        return
    q, d = act.quantize(x)
    assert np.all(np.abs(q.astype(np.int64)) <= 127)
    for m in range(2):
        k = int(np.argmax(np.abs(x[m])))
        assert abs(int(q[m, k])) == 127 and np.sign(q[m, k]) == np.sign(x[m, k])
        err = np.abs(q[m].astype(np.float64) * np.float64(d[m]) - x[m].astype(np.float64))
        assert np.all(err <= 0.5 * np.float64(d[m]) * (1 + 1e-5) + 1e-6 * np.abs(x[m]))


def test_group_sums_and_planes_bruteforce():
    rng = np.random.default_rng(5)
    q = rng.integers(-127, 128, size=(3, 256)).astype(np.int8)
    S = act.group_sums(q, 32)
    for m in range(3):
        for g in range(8):
            assert S[m, g] == sum(int(v) for v in q[m, 32 * g:32 * g + 32])
    P = act.planes(q)                       # [8, M, K/32]
    for m in range(3):
        for k in [0, 31, 32, 200, 255]:
            byte = int(q[m, k]) & 0xFF
            for j in range(8):
                assert (int(P[j, m, k // 32]) >> (k % 32)) & 1 == (byte >> j) & 1
