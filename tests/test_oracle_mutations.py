"""Planted mistakes: each test mutates one step of the oracle (on the CPU) and
checks that one of the pins fails.  This shows the pins can tell a plausible
error from the intended arithmetic."""
import numpy as np
import pytest

from oracle import act, bitserial, weights as ow
from oracle import common
import oracle.gemv as og
import test_oracle_bitplanes as tb
import test_oracle_gemv as tg
import test_oracle_weights as tw


def test_mutation_sign_plane_weight(monkeypatch):
    # sign plane weighted +128 instead of -128
    monkeypatch.setattr(bitserial, "ACT_PLANE_WEIGHTS",
                        np.array([1, 2, 4, 8, 16, 32, 64, 128], dtype=np.int64))
    with pytest.raises(AssertionError):
        tb.test_act_planes_exhaustive_twos_complement()


def test_mutation_msb_first_packing(monkeypatch):
    def pack_msb(bits):
        bits = np.asarray(bits, dtype=np.uint64)
        K = bits.shape[-1]
        b = bits.reshape(bits.shape[:-1] + (K // 32, 32))
        return (b << np.arange(31, -1, -1, dtype=np.uint64)).sum(-1).astype(np.uint32)
    monkeypatch.setattr(bitserial, "pack_bits", pack_msb)
    with pytest.raises(AssertionError):
        tb.test_pack_bits_lsb_first_positions()


def test_mutation_sign_tie(monkeypatch):
    monkeypatch.setattr(common, "sign_pm1",
                        lambda v: np.where(np.asarray(v) > 0, 1, -1).astype(np.int8))
    monkeypatch.setattr(tb, "sign_pm1", common.sign_pm1)
    with pytest.raises(AssertionError):
        tb.test_sign_tie_rule()


def test_mutation_round_half_away(monkeypatch):
    real = np.rint

    def quantize_half_away(x_f32):
        x = np.asarray(x_f32, dtype=np.float32)
        amax = np.max(np.abs(x), axis=1)
        q = np.zeros(x.shape, np.int8)
        d = np.zeros(x.shape[0], np.float32)
        for m in range(x.shape[0]):
            if amax[m] == 0:
                continue
            s = np.float32(127.0) / amax[m]
            p = x[m] * s
            q[m] = np.clip(np.sign(p) * np.floor(np.abs(p) + 0.5), -127, 127)
            d[m] = amax[m] / np.float32(127.0)
        return q, d
    assert real is np.rint
    monkeypatch.setattr(act, "quantize", quantize_half_away)
    with pytest.raises(AssertionError):
        tb.test_act_quant_hand_cases()


def test_mutation_ternary_absmax(monkeypatch):
    def absmax(W):
        W = np.asarray(W, dtype=np.float32)
        gamma = np.float32(np.max(np.abs(W)))
        return np.clip(np.rint(W / gamma), -1, 1).astype(np.int8), gamma
    monkeypatch.setattr(ow, "quantize_ternary", absmax)
    with pytest.raises(AssertionError):
        tw.test_ternary_zero_fraction_gaussian()


def test_mutation_w2a8_zero_point_sign(monkeypatch):
    real = ow.quantize_w2a8

    def flipped(W, group=128):
        q, delta, zero = real(-np.asarray(W), group)     # z computed from +lo
        return q, delta, zero
    monkeypatch.setattr(ow, "quantize_w2a8", flipped)
    with pytest.raises(AssertionError):
        tw.test_w2a8_hand_case()


def test_mutation_bvsr_dropped_bitvector(monkeypatch):
    def points3(cache):
        c = np.asarray(cache, dtype=np.float32).astype(np.float64)
        codes = np.arange(16)
        v = np.repeat(c[:, 4:5], 16, axis=1)
        for k in range(3):                               # c3 term dropped
            bit = ((codes >> k) & 1).astype(bool)
            v = np.where(bit[None, :], v + c[:, k:k + 1], v)
        return v
    monkeypatch.setattr(ow, "bvsr_points", points3)
    with pytest.raises(AssertionError):
        tw.test_bvsr_ratio_two_is_uniform_grid()


def test_mutation_rabit_transposed_scales(monkeypatch):
    # h applied per row and g per column (operands swapped): breaks the
    # factorization pin on a non-square layer
    def deq_swapped(B, g, h, n0=0, n1=None):
        n1 = B.shape[1] if n1 is None else n1
        out = np.zeros((n1 - n0, B.shape[2]))
        for p in range(B.shape[0]):
            hh = np.resize(h[p].astype(np.float64), n1 - n0)
            gg = np.resize(g[p].astype(np.float64), B.shape[2])
            out += hh[:, None] * B[p, n0:n1] * gg[None, :]
        return out
    monkeypatch.setattr(og, "deq_rabit", deq_swapped)
    with pytest.raises(AssertionError):
        tg.test_rabit_gemv_and_factorization()


def test_mutation_w2a8_dropped_zero_point_term(monkeypatch):
    def no_zero(A, S, delta, zero, d):
        dl = delta.astype(np.float64)[None]
        return np.asarray(d, np.float64)[:, None] * (dl * A.astype(np.float64)).sum(-1)
    monkeypatch.setattr(og, "w2a8_from_int", no_zero)
    with pytest.raises(AssertionError):
        tg.test_w2a8_int_zero_point_identity()


def test_mutation_hgf_relu_instead_of_silu(monkeypatch):
    import test_oracle_hgf as th
    monkeypatch.setattr(og, "silu", lambda z: np.maximum(np.asarray(z, np.float64), 0.0))
    with pytest.raises(AssertionError):
        th.test_lora_correction_hand_case()


def test_mutation_hgf_sigmoid_sign(monkeypatch):
    import test_oracle_hgf as th
    monkeypatch.setattr(og, "silu", lambda z: np.asarray(z, np.float64) / (1.0 + np.exp(np.asarray(z, np.float64))))
    with pytest.raises(AssertionError):
        th.test_silu_special_values()


def test_mutation_hgf_ungated(monkeypatch):
    import test_oracle_hgf as th
    monkeypatch.setattr(og, "lora_gate", lambda alpha: np.float64(alpha))
    with pytest.raises(AssertionError):
        th.test_lora_correction_hand_case()


def test_mutation_hgf_quantized_input(monkeypatch):
    # feeding the correction the quantized activation q instead of x
    import test_oracle_hgf as th
    orig = og.gemv_hgf

    def wrong(T, gamma, q, d, x, A, B, alpha):
        return orig(T, gamma, q, d, q.astype(np.float64), A, B, alpha)
    monkeypatch.setattr(og, "gemv_hgf", wrong)
    with pytest.raises(AssertionError):
        th.test_gemv_hgf_hand_case()


def test_mutation_bit_balance_asymmetric_grid(monkeypatch):
    # the four-level INT2 grid {-2,-1,0,1} in place of the balanced five levels
    import test_oracle_bitbalance as tbb
    orig = ow.quantize_bit_balance

    def four_level(W, group=128):
        c, d, z = orig(W, group)
        return np.minimum(c, 3).astype(np.uint8), d, z
    monkeypatch.setattr(ow, "quantize_bit_balance", four_level)
    with pytest.raises(AssertionError):
        tbb.test_mirror_symmetry()


def test_mutation_bit_balance_step_from_range(monkeypatch):
    # the asymmetric (hi - lo) / 4 step instead of max|W| / 2
    import test_oracle_bitbalance as tbb

    def range_step(W, group=128):
        W = np.asarray(W, np.float32)
        N, K = W.shape
        Wg = W.reshape(N, K // group, group).astype(np.float64)
        d16 = common.to_f16((Wg.max(-1) - Wg.min(-1)) / 4.0)
        t = np.clip(np.rint(Wg / np.where(d16 == 0, 1.0, d16.astype(np.float64))[..., None]), -2, 2)
        return (t + 2).reshape(N, K).astype(np.uint8), d16, np.full(d16.shape, 2.0, np.float16)
    monkeypatch.setattr(ow, "quantize_bit_balance", range_step)
    with pytest.raises(AssertionError):
        tbb.test_hand_case()
