"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: integer results (activation codes, planes, group sums, int32 partial
sums) bit-exact; fp32 outputs within |y - y_ref| <= 2e-3 * sum_k |w^ x^| per
output, the oracle's fp64 reference computed from the same logical form.
Sizes: small ragged cases spanning several tiles and splits, and the
workload sizes (all outputs where the oracle is cheap, sampled rows where
it is not).
"""
import numpy as np
import pytest

import bit_plane_gemv_amd as bq
from oracle import act as oact, gemv as og, weights as ow, bitserial
import synth
from gpuhelp import (assert_within, dev_blob, parse_act, qm_from_q, quantize_act_dev, run_gemv, say, to_dev, torch,
                     workspace)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ======================================================= activation quantizer
def _check_act(x_store, x_f32, M, K, abits=8):
    act, got = quantize_act_dev(x_store, M, K, abits)
    _act_matches(got, x_f32, K, abits)
    return act


def _act_matches(got, x_f32, K, abits=8):
    """The parsed activation sections equal the oracle's quantization."""
    q, d = oact.quantize(x_f32, abits)
    assert np.array_equal(got["q"][:, :K], q), "q"
    assert np.all(got["q"][:, K:] == 0), "q padding"
    assert np.array_equal(got["d"].view(np.uint32), d.view(np.uint32)), "d"
    Kw_real = K // 32
    pl = oact.planes(q)                                    # [8, M, K/32]
    assert np.array_equal(got["planes"][:, :Kw_real, :], pl.transpose(1, 2, 0)), "planes"
    assert np.all(got["planes"][:, Kw_real:, :] == 0), "planes padding"
    assert np.array_equal(got["S"][:, :Kw_real], oact.group_sums(q, 32)), "S"
    assert np.all(got["S"][:, Kw_real:] == 0)
    assert np.array_equal(got["qm"], qm_from_q(got["q"])), "qm (the matrix-core order of q)"
    amax = np.max(np.abs(np.asarray(x_f32, np.float32)), axis=1)
    assert np.array_equal(got["amax"].view(np.uint32), amax.view(np.uint32)), "amax"


@pytest.mark.parametrize("M,K", [(1, 4096), (1, 224), (16, 512), (64, 11008), (3, 32)])
def test_act_quant_bitexact_bf16(M, K):
    say("act_quant bf16", M, K)
    bits, xf = synth.random_bf16(np.random.default_rng(M * 7 + K), (M, K))
    if M > 2:
        bits[1] = 0                                           # an all-zero token
        xf[1] = 0
    _check_act(bits, xf, M, K)


@pytest.mark.parametrize("M,K,f32", [(2, 16416, False), (3, 32768, True), (1, 1 << 20, False)])
def test_act_quant_long_rows(M, K, f32):
    # K above 16384: amax from a pass of its own, then every workgroup reads
    # only its own inputs; the sections are the same bits
    say("act_quant long rows", M, K, f32)
    if f32:
        xf = synth.gaussian_f32(np.random.default_rng(K + M), (M, K), 3.0)
        bits = xf
    else:
        bits, xf = synth.random_bf16(np.random.default_rng(K + M), (M, K))
    xf[0, K - 1] = bits[0, K - 1] = 0                         # amax elsewhere in the row
    _check_act(bits, xf, M, K)


@pytest.mark.parametrize("abits", [2, 3, 4, 6, 7])
def test_act_quant_bits_bitexact(abits):
    say("act_quant bits", abits)
    M, K = 5, 1056
    bits, xf = synth.random_bf16(np.random.default_rng(abits), (M, K))
    bits[2] = 0
    xf[2] = 0
    _check_act(bits, xf, M, K, abits)


def test_act_quant_ties_and_f32():
    say("act_quant ties f32")
    K = 256
    x = np.zeros((4, K), dtype=np.float32)
    x[0, 0] = 127.0                                           # s = 1: exact .5 ties
    x[0, 1:9] = [2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5, 126.5]
    x[1, :] = np.linspace(-3, 3, K, dtype=np.float32)
    x[2, 5] = -1e-30                                          # tiny single value
    x[3] = synth.gaussian_f32(np.random.default_rng(1), K, 1e4)
    _check_act(x, x, 4, K)


# ================================================================ sign / RaBiT
def _sign_case(N, K, x_kind="f32", seed=0):
    W = synth.gaussian_f32(np.random.default_rng(seed), (N, K), 1.0)
    B, alpha = ow.quantize_sign(W)
    if x_kind == "f32":
        x = synth.gaussian_f32(np.random.default_rng(seed + 1), (1, K), 1.0)
        xs = x
    else:
        xs, x = synth.random_bf16(np.random.default_rng(seed + 1), (1, K))
    desc = bq.wdesc(bq.SIGN1, N, K)
    blob = bq.pack_weights(desc, sign=B, alpha=alpha)
    y = run_gemv(desc, dev_blob(blob), to_dev(xs[0]), bq.DT_F32 if x_kind == "f32" else bq.DT_BF16)
    y_ref, tol = og.gemv_sign(B, alpha, x)
    return assert_within(y, y_ref, tol, f"sign {N}x{K}")


@pytest.mark.parametrize("N,K,xk", [(256, 256, "f32"), (200, 224, "f32"), (1000, 1056, "bf16"),
                                    (64, 32, "f32")])
def test_sign_gemv(N, K, xk):
    say("sign", N, K, xk)
    _sign_case(N, K, xk)


# ===================================================== fully binary (XNOR)
def _binarize_dev(x_store, M, K):
    t = torch()
    x = to_dev(x_store)
    dt = bq.DT_F32 if x_store.dtype == np.float32 else bq.DT_BF16
    act = t.full((bq.binact_size(M, K),), 0x5A, dtype=t.uint8, device="cuda")  # poison
    bq.binarize_act(x, dt, M, K, act)
    t.cuda.synchronize()
    L = bq.binact_layout(M, K)
    h = act.cpu().numpy()
    bits = h[:4 * M * L["Kw"]].view(np.uint32).reshape(M, L["Kw"])
    beta = h[L["off_beta"]:L["off_beta"] + 4 * M].view(np.float32)
    return act, bits, beta


def _xnor_case(N, K, M, x_store, x_f32, seed=0, rows=None):
    W = synth.gaussian_f32(np.random.default_rng(seed), (N, K), 1.0)
    B, alpha = ow.quantize_sign(W)
    xb, beta = oact.binarize(x_f32)
    act, bits, beta_dev = _binarize_dev(x_store, M, K)
    assert np.array_equal(bits, oact.binary_words(xb, bq.binact_layout(M, K)["Kp"])), "sign words"
    assert np.all(np.abs(beta_dev - beta) <= 1e-6 * beta + 1e-30), "beta"
    desc = bq.wdesc(bq.SIGN1, N, K)
    bd = dev_blob(bq.pack_weights(desc, sign=B, alpha=alpha))
    r = np.arange(N) if rows is None else rows
    t = torch()
    Yd = t.full((M * N,), -1, dtype=t.int32, device="cuda")
    yd = t.full((M * N,), float("nan"), dtype=t.float32, device="cuda")
    for buf, flags in ((Yd, bq.F_ACC_INT32), (yd, 0)):
        if M == 1:
            bq.gemv(desc, bd, act, bq.DT_BINARY, buf, None, flags=flags)
        else:
            bq.gemm_smallM(desc, bd, act, M, buf, None, flags=flags)
    t.cuda.synchronize()
    Y = Yd.cpu().numpy().reshape(M, N)
    assert np.array_equal(Y[:, r], og.xnor_int(B[r], xb)), "xnor Y"
    # the float output against the oracle, with the device's beta (an fp32 sum)
    y_ref, tol = og.gemv_xnor(B[r], alpha[r], xb, beta_dev.astype(np.float64))
    return assert_within(yd.cpu().numpy().reshape(M, N)[:, r], y_ref, tol, f"xnor {N}x{K} M={M}")


@pytest.mark.parametrize("N,K,M", [(256, 256, 1), (70, 224, 1), (200, 4096, 1), (130, 1056, 5),
                                   (64, 32, 1), (300, 40960, 1), (1000, 2048, 64)])
def test_xnor_gemv(N, K, M):
    say("xnor", N, K, M)
    xs, xf = synth.random_bf16(np.random.default_rng(N + M), (M, K))
    xs[:, 0] = 0x8000                                   # -0.0 -> +1
    xf[:, 0] = -0.0
    _xnor_case(N, K, M, xs, xf, seed=N)


def test_xnor_gemv_workload_and_batch_invariance():
    N, K = 11008, 4096
    say("xnor workload", N, K)
    xs, xf = synth.random_bf16(np.random.default_rng(77), (4, K))
    rows = np.sort(np.random.default_rng(1).choice(N, 512, replace=False))
    _xnor_case(N, K, 4, xs, xf, seed=9, rows=rows)
    # token 2 alone equals token 2 of the batch, bit for bit
    W = synth.gaussian_f32(np.random.default_rng(9), (N, K), 1.0)
    B, alpha = ow.quantize_sign(W)
    desc = bq.wdesc(bq.SIGN1, N, K)
    bd = dev_blob(bq.pack_weights(desc, sign=B, alpha=alpha))
    t = torch()
    act4, _, _ = _binarize_dev(xs, 4, K)
    act1, _, _ = _binarize_dev(xs[2:3], 1, K)
    y4 = t.empty(4 * N, dtype=t.float32, device="cuda")
    y1 = t.empty(N, dtype=t.float32, device="cuda")
    bq.gemm_smallM(desc, bd, act4, 4, y4, None)
    bq.gemv(desc, bd, act1, bq.DT_BINARY, y1, None)
    t.cuda.synchronize()
    assert np.array_equal(y4.cpu().numpy().reshape(4, N)[2].view(np.uint32), y1.cpu().numpy().view(np.uint32))


def _rabit_case(N, K, P, W=None, xs=None, x=None, seed=0):
    if W is None:
        W = synth.gaussian_f32(np.random.default_rng(seed), (N, K), 0.02)
    if xs is None:
        xs, x = synth.random_bf16(np.random.default_rng(seed + 1), (1, K))
    B, g, h = ow.quantize_rabit(W, paths=P)
    desc = bq.wdesc(bq.RABIT, N, K, planes=P)
    blob = bq.pack_weights(desc, sign=B, g=g, h=h)
    y = run_gemv(desc, dev_blob(blob), to_dev(xs[0]), bq.DT_BF16)
    y_ref, tol = og.gemv_rabit(B, g, h, x)
    return assert_within(y, y_ref, tol, f"rabit {N}x{K} P={P}")


@pytest.mark.parametrize("N,K", [(300, 416), (64, 128), (520, 2048)])
@pytest.mark.parametrize("P", [1, 2, 3])
def test_rabit_gemv_small(N, K, P):
    say("rabit", N, K, P)
    _rabit_case(N, K, P)


@pytest.mark.parametrize("N,K,P", [(200, 32256, 2), (256, 32768, 1), (70, 64512, 1), (136, 20096, 3)])
def test_rabit_gemv_many_splits(N, K, P):
    # 63 splits (the most the split-k arrival count holds), 8 k blocks per
    # split, and the largest K of the float formats
    say("rabit many splits", N, K, P)
    _rabit_case(N, K, P, seed=3)


def test_rabit_split_k_deterministic_and_workspace_reuse():
    """The fixed-point split-k sum does not depend on the arrival order:
    repeated calls on one workspace give bit-identical y, and each call
    leaves the workspace words at zero for the next."""
    N, K = 11008, 4096
    say("rabit determinism", N, K)
    t = torch()
    W = synth.weights("rabit", 1, N, K)
    xs, x = synth.activations("rabit", 1, 1, K)
    B, g, h = ow.quantize_rabit(W, paths=2)
    desc = bq.wdesc(bq.RABIT, N, K, planes=2)
    bd = dev_blob(bq.pack_weights(desc, sign=B, g=g, h=h))
    xd = to_dev(xs[0])
    ws = workspace(desc)
    assert ws.numel() > 0
    outs = []
    for _ in range(5):
        y = t.full((N,), float("nan"), dtype=t.float32, device="cuda")
        bq.gemv(desc, bd, xd, bq.DT_BF16, y, ws)
        t.cuda.synchronize()
        outs.append(y.cpu().numpy())
        assert not ws.any().item(), "split-k words not reset"
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    y_ref, tol = og.gemv_rabit(B, g, h, x)
    assert_within(outs[0][None, :], y_ref, tol, "rabit determinism")


@pytest.mark.parametrize("N,K,P", [(12352, 256, 2), (28672, 384, 1), (16, 4096, 2), (4160, 1024, 3)])
def test_rabit_gemv_row_ranges(N, K, P):
    # many row groups (the last one partial), a layer of one row tile, and
    # three paths on a ragged N
    say("rabit row ranges", N, K, P)
    _rabit_case(N, K, P, seed=4)


@pytest.mark.parametrize("fmt", ["rabit", "sign"])
def test_float_gemv_nan_input_propagates(fmt):
    """A NaN input makes every output row NaN (each row adds +-h x_k for every
    k; the split-k bound is NaN too); the rows of a NaN-free call are finite."""
    N, K = 300, 1056
    say("nan propagation", fmt)
    t = torch()
    W = synth.gaussian_f32(np.random.default_rng(5), (N, K), 0.02)
    x = synth.gaussian_f32(np.random.default_rng(6), (1, K), 1.0)[0].copy()
    if fmt == "rabit":
        B, g, h = ow.quantize_rabit(W, paths=2)
        desc = bq.wdesc(bq.RABIT, N, K, planes=2)
        blob = bq.pack_weights(desc, sign=B, g=g, h=h)
    else:
        B, alpha = ow.quantize_sign(W)
        desc = bq.wdesc(bq.SIGN1, N, K)
        blob = bq.pack_weights(desc, sign=B, alpha=alpha)
    bd = dev_blob(blob)
    y0 = run_gemv(desc, bd, to_dev(x), bq.DT_F32)
    assert np.all(np.isfinite(y0))
    x[777] = np.nan
    y1 = run_gemv(desc, bd, to_dev(x), bq.DT_F32)
    assert np.all(np.isnan(y1))


def test_rabit_gemv_svid_refined_blob():
    """The refined RaBiT decomposition (library packer, 20 Gauss-Seidel sweeps)
    runs through the same GEMV; parity from the logical form the oracle reads
    back out of the blob."""
    from oracle import layout
    N, K = 4096, 4096
    say("rabit svid blob", N, K)
    W = synth.weights("rabit", 0, N, K)
    xs, x = synth.activations("rabit", 0, 1, K)
    desc = bq.wdesc(bq.RABIT, N, K, planes=2)
    blob = bq.quantize_weights(desc, W, svid_sweeps=20)
    L = layout.unpack(blob)
    y = run_gemv(desc, dev_blob(blob), to_dev(xs[0]), bq.DT_BF16)
    y_ref, tol = og.gemv_rabit(L["B"], L["g"], L["h"], x)
    assert_within(y, y_ref, tol, "rabit svid")


@pytest.mark.parametrize("shape_idx", [0, 1, 2])
def test_rabit_gemv_workload(shape_idx):
    N, K = synth.CONFIGS["rabit"]["shapes"][shape_idx]
    say("rabit workload", N, K)
    W = synth.weights("rabit", shape_idx, N, K)
    xs, x = synth.activations("rabit", shape_idx, 1, K)
    r = _rabit_case(N, K, 2, W, xs, x)
    say("max err/tol", r)


# ================================================================== ternary
def _int_case(fmt, N, K, M, W, xs, xf, rows=None, extra=None):
    """Quantize (oracle), pack (library), run the GPU both in ACC and float
    mode, compare.  rows: subset of output rows checked against the oracle."""
    q, d = oact.quantize(xf)
    act, _ = quantize_act_dev(xs, M, K)
    desc = bq.wdesc(fmt, N, K)
    r = np.arange(N) if rows is None else rows
    if fmt == bq.TERNARY:
        T, gamma = ow.quantize_ternary(W)
        blob = bq.pack_weights(desc, tern=T, gamma=gamma)
        bd = dev_blob(blob)
        Yi = run_gemv(desc, bd, act, bq.DT_ACT, M, bq.F_ACC_INT32, M * N).reshape(M, N)
        Y_ref = og.ternary_int(T[r], q)
        assert np.array_equal(Yi[:, r], Y_ref), "ternary Y_int"
        y = run_gemv(desc, bd, act, bq.DT_ACT, M)
        y_ref, tol = og.gemv_ternary(T[r], gamma, q, d)
    elif fmt == bq.W2A8:
        qw, delta, zero = ow.quantize_w2a8(W)
        blob = bq.pack_weights(desc, code=qw, delta=delta, zero=zero)
        bd = dev_blob(blob)
        G = K // 128
        A = run_gemv(desc, bd, act, bq.DT_ACT, M, bq.F_ACC_INT32, M * N * G).reshape(M, N, G)
        assert np.array_equal(A[:, r], og.w2a8_int(qw[r], q)), "w2a8 A"
        y = run_gemv(desc, bd, act, bq.DT_ACT, M)
        y_ref, tol = og.gemv_w2a8(qw[r], delta[r], zero[r], q, d)
    else:
        code, idx, cache = extra
        blob = bq.pack_weights(desc, code=code, idx=idx, cache=cache)
        bd = dev_blob(blob)
        G = K // 32
        P = run_gemv(desc, bd, act, bq.DT_ACT, M, bq.F_ACC_INT32, M * N * G * 4).reshape(M, N, G, 4)
        assert np.array_equal(P[:, r], og.bvsr_int(code[r], q)), "bvsr P"
        y = run_gemv(desc, bd, act, bq.DT_ACT, M)
        y_ref, tol = og.gemv_bvsr(code[r], idx[r], cache, q, d)
    return assert_within(y[:, r], y_ref, tol, f"fmt {fmt} {N}x{K} M={M}"), y


@pytest.mark.parametrize("N,K", [(512, 512), (2048, 512), (512, 2048), (70, 224), (4096, 4096)])
@pytest.mark.parametrize("M", [1, 16])
def test_ternary(N, K, M):
    say("ternary", N, K, M)
    W = synth.gaussian_f32(np.random.default_rng(N + K), (N, K), 0.02)
    xs, xf = synth.random_bf16(np.random.default_rng(M), (M, K))
    _int_case(bq.TERNARY, N, K, M, W, xs, xf)


# ===================================================================== W2A8
@pytest.mark.parametrize("N,K", [(70, 256), (130, 1152)])
@pytest.mark.parametrize("M", [1, 4, 64])
def test_w2a8_small(N, K, M):
    say("w2a8 small", N, K, M)
    W = synth.gaussian_f32(np.random.default_rng(N * K), (N, K), 0.02)
    xs, xf = synth.activations("w2a8", 0, M, K)
    _int_case(bq.W2A8, N, K, M, W, xs, xf)


@pytest.mark.parametrize("shape_idx", [0, 1, 2])
@pytest.mark.parametrize("M", [1, 4, 8, 16, 64])
def test_w2a8_workload(shape_idx, M):
    N, K = synth.CONFIGS["w2a8"]["shapes"][shape_idx]
    say("w2a8 workload", N, K, M)
    W = synth.weights("w2a8", shape_idx, N, K)
    xs, xf = synth.activations("w2a8", shape_idx, M, K)
    rows = None if M == 1 else np.sort(np.random.default_rng(M).choice(N, 384, replace=False))
    _int_case(bq.W2A8, N, K, M, W, xs, xf, rows=rows)


def test_w2a8_batch_invariance_and_determinism():
    """Run to run, and for a token whatever its place in a batch of the same
    size, the output bits are the same (same kernel, same launch shape).
    Other batch sizes may run another kernel or launch shape (M = 1 the VALU
    kernel, 16 and 40 different matrix-core shapes), which add the fp32 group
    terms in another order: there the outputs agree within the tolerance,
    and the exact integer partials agree bit for bit."""
    N, K = 11008, 4096
    say("w2a8 batch invariance", N, K)
    W = synth.weights("w2a8", 1, N, K)
    xs, xf = synth.activations("w2a8", 1, 16, K)
    qw, delta, zero = ow.quantize_w2a8(W)
    desc = bq.wdesc(bq.W2A8, N, K)
    bd = dev_blob(bq.pack_weights(desc, code=qw, delta=delta, zero=zero))
    act16, _ = quantize_act_dev(xs, 16, K)
    ws = workspace(desc, 16)
    y16a = run_gemv(desc, bd, act16, bq.DT_ACT, 16, ws=ws)
    y16b = run_gemv(desc, bd, act16, bq.DT_ACT, 16, ws=ws)
    assert np.array_equal(y16a.view(np.uint32), y16b.view(np.uint32)), "run-to-run"
    perm = np.roll(np.arange(16), 5)
    act16p, _ = quantize_act_dev(np.ascontiguousarray(xs[perm]), 16, K)
    y16p = run_gemv(desc, bd, act16p, bq.DT_ACT, 16, ws=ws)
    assert np.array_equal(y16p.view(np.uint32), y16a[perm].view(np.uint32)), "token order within a batch"
    q, d = oact.quantize(xf)
    y_ref, tol = og.gemv_w2a8(qw, delta, zero, q, d)
    assert_within(y16a, y_ref, tol, "M = 16 against the oracle")
    for m in (0, 9, 15):
        sub = np.ascontiguousarray(xs[[(m + 5) % 16, m]])
        act2, _ = quantize_act_dev(sub, 2, K)
        y2 = run_gemv(desc, bd, act2, bq.DT_ACT, 2, ws=ws)
        assert_within(y2[1], y16a[m].astype(np.float64), tol[m], f"token {m}: M = 2 against M = 16")
        assert_within(y2[1], y_ref[m], tol[m], f"token {m}: M = 2 against the oracle")
    x40 = np.ascontiguousarray(np.concatenate([xs, xs, xs[:8]]))
    act40, _ = quantize_act_dev(x40, 40, K)
    y40 = run_gemv(desc, bd, act40, bq.DT_ACT, 40, ws=ws)
    assert_within(y40[16:32], y16a.astype(np.float64), tol, "M = 40 against M = 16")
    assert np.array_equal(y40[0:16].view(np.uint32), y40[16:32].view(np.uint32)), "same tokens, same batch"
    G = K // 128
    A16 = run_gemv(desc, bd, act16, bq.DT_ACT, 16, bq.F_ACC_INT32, 16 * N * G).reshape(16, N, G)
    A40 = run_gemv(desc, bd, act40, bq.DT_ACT, 40, bq.F_ACC_INT32, 40 * N * G).reshape(40, N, G)
    assert np.array_equal(A40[16:32], A16), "partials, M = 40 against M = 16"
    ws1 = workspace(desc, 1)
    for m in (0, 15):
        act1, _ = quantize_act_dev(xs[m:m + 1], 1, K)
        A1 = run_gemv(desc, bd, act1, bq.DT_ACT, 1, bq.F_ACC_INT32, N * G, ws=ws1).reshape(N, G)
        assert np.array_equal(A1, A16[m]), f"token {m} partials"


# ===================================================================== WnAm
def _wnam_case(N, K, M, n, m, W, xs, xf, rows=None, balanced=False):
    """n-bit weights (oracle RTN, or the oracle's bit-balance grid; library
    packer) x m-bit activations (library quantizer, checked against the
    oracle's): exact group partials A and the float output within tolerance."""
    q, d = oact.quantize(xf, m)
    act, got = quantize_act_dev(xs, M, K, m)
    assert np.array_equal(got["q"][:, :K], q) and np.array_equal(got["d"].view(np.uint32), d.view(np.uint32))
    qw, delta, zero = ow.quantize_bit_balance(W) if balanced else ow.quantize_wnam(W, n)
    desc = bq.wdesc(bq.WNAM, N, K, planes=n, abits=m)
    bd = dev_blob(bq.pack_weights(desc, code=qw, delta=delta, zero=zero))
    r = np.arange(N) if rows is None else rows
    G = K // 128
    A = run_gemv(desc, bd, act, bq.DT_ACT, M, bq.F_ACC_INT32, M * N * G).reshape(M, N, G)
    assert np.array_equal(A[:, r], og.w2a8_int(qw[r], q)), f"wnam A n={n} m={m}"
    y = run_gemv(desc, bd, act, bq.DT_ACT, M)
    y_ref, tol = og.gemv_w2a8(qw[r], delta[r], zero[r], q, d)
    return assert_within(y[:, r], y_ref, tol, f"wnam W{n}A{m} {N}x{K} M={M}"), y


@pytest.mark.parametrize("n,m", [(1, 8), (2, 4), (3, 3), (4, 4), (4, 2), (3, 6), (2, 8)])
@pytest.mark.parametrize("N,K,M", [(200, 512, 1), (70, 1152, 4), (130, 4096, 1)])
def test_wnam_gemv(n, m, N, K, M):
    say("wnam", n, m, N, K, M)
    W = synth.gaussian_f32(np.random.default_rng(N + K + n), (N, K), 0.02)
    xs, xf = synth.activations("w2a8", 0, M, K)
    _wnam_case(N, K, M, n, m, W, xs, xf)


def test_wnam_w2_a8_equals_w2a8():
    """W2A8 through the WnAm kernel (n = 2, m = 8) gives the W2A8 kernel's
    output bit for bit."""
    N, K = 1000, 2048
    say("wnam W2A8 vs w2a8", N, K)
    W = synth.gaussian_f32(np.random.default_rng(11), (N, K), 0.02)
    xs, xf = synth.activations("w2a8", 0, 1, K)
    qw, delta, zero = ow.quantize_w2a8(W)
    act, _ = quantize_act_dev(xs, 1, K)
    dw = bq.wdesc(bq.W2A8, N, K)
    dn = bq.wdesc(bq.WNAM, N, K, planes=2, abits=8)
    y1 = run_gemv(dw, dev_blob(bq.pack_weights(dw, code=qw, delta=delta, zero=zero)), act, bq.DT_ACT)
    y2 = run_gemv(dn, dev_blob(bq.pack_weights(dn, code=qw, delta=delta, zero=zero)), act, bq.DT_ACT)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("n,m,M", [(4, 4, 1), (3, 8, 1), (2, 4, 16)])
def test_wnam_workload(n, m, M):
    N, K = 11008, 4096
    say("wnam workload", n, m, N, K, M)
    W = synth.weights("w2a8", 1, N, K)
    xs, xf = synth.activations("w2a8", 1, M, K)
    rows = np.sort(np.random.default_rng(n * m).choice(N, 512, replace=False))
    _wnam_case(N, K, M, n, m, W, xs, xf, rows=rows)


# ===================================================================== BVSR
def _span_matched_encoding(W, cache, row_chunk=256):
    """A valid BVSR encoding built by the oracle for large parity inputs: each
    group takes the set with ratio index 8 whose span is nearest the group's
    range, then nearest-point codes (oracle bvsr_encode).  Not the exhaustive
    search (too slow at full size); the GEMV result does not depend on which
    valid encoding is fed to both sides."""
    N, K = W.shape
    G = K // 32
    L = -2.0 * cache[16 * 8:16 * 8 + 16, 4].astype(np.float64)
    code = np.empty((N, K), np.uint8)
    idx = np.empty((N, G), np.uint8)
    for n0 in range(0, N, row_chunk):
        w = W[n0:n0 + row_chunk].astype(np.float64).reshape(-1, G, 32)
        span = w.max(-1) - w.min(-1)
        j = np.argmin(np.abs(span[..., None] - L[None, None, :]), axis=-1)
        idx[n0:n0 + row_chunk] = (16 * 8 + j).astype(np.uint8)
        code[n0:n0 + row_chunk], _ = ow.bvsr_encode(W[n0:n0 + row_chunk], cache, idx[n0:n0 + row_chunk])
    return code, idx


@pytest.mark.parametrize("N,K", [(128, 512), (70, 224)])
def test_bvsr_small_exhaustive(N, K):
    say("bvsr small", N, K)
    W = synth.gaussian_f32(np.random.default_rng(N + K), (N, K), 0.015)
    cache = ow.bvsr_cache(W)
    code, idx, _ = ow.bvsr_search(W, cache)
    xs, xf = synth.random_bf16(np.random.default_rng(5), (1, K))
    _int_case(bq.BVSR4, N, K, 1, W, xs, xf, extra=(code, idx, cache))


@pytest.mark.parametrize("shape_idx", [0, 1])
def test_bvsr_workload(shape_idx):
    N, K = synth.CONFIGS["bvsr"]["shapes"][shape_idx]
    say("bvsr workload", N, K)
    W = synth.weights("bvsr", shape_idx, N, K)
    cache = ow.bvsr_cache(W) if shape_idx == 0 else ow.bvsr_cache(W[:4096])
    if shape_idx == 0:
        code, idx = _span_matched_encoding(W, cache)
        rows = None
    else:
        # realistic encoding on the checked rows, random valid codes elsewhere
        rng = np.random.default_rng(7)
        rows = np.sort(rng.choice(N, 512, replace=False))
        code = rng.integers(0, 16, (N, K), dtype=np.uint8)
        idx = rng.integers(0, 256, (N, K // 32), dtype=np.uint8)
        c_r, i_r = _span_matched_encoding(W[rows], cache)
        code[rows], idx[rows] = c_r, i_r
    xs, xf = synth.activations("bvsr", shape_idx, 1, K)
    _int_case(bq.BVSR4, N, K, 1, W, xs, xf, rows=rows, extra=(code, idx, cache))


# ======================================================= AND+popcount on GPU
@pytest.mark.parametrize("fmt", [bq.W2A8, bq.BVSR4, bq.TERNARY])
@pytest.mark.parametrize("c", [0, 45, 127])
def test_single_element_tables_on_gpu(fmt, c):
    """Exhaustive (weight code) x (int8 activation) products through the GPU
    AND+popcount path: row n holds code n at channel c, token m holds q = v_m
    at channel c (and 127 elsewhere on one channel so that amax = 127, s = 1)."""
    K = 256
    say("single-element tables", fmt, c)
    e = 255 if c != 255 else 0
    ncodes = {bq.W2A8: 4, bq.BVSR4: 16, bq.TERNARY: 3}[fmt]
    Wc = np.zeros((ncodes, K), np.int64)
    Wc[:, c] = np.arange(ncodes) - (1 if fmt == bq.TERNARY else 0)
    desc = bq.wdesc(fmt, ncodes, K)
    if fmt == bq.W2A8:
        blob = bq.pack_weights(desc, code=Wc.astype(np.uint8), delta=np.ones((ncodes, 2), np.float16),
                               zero=np.zeros((ncodes, 2), np.float16))
    elif fmt == bq.BVSR4:
        blob = bq.pack_weights(desc, code=Wc.astype(np.uint8), idx=np.zeros((ncodes, 8), np.uint8),
                               cache=np.zeros((256, 5), np.float32))
    else:
        blob = bq.pack_weights(desc, tern=Wc.astype(np.int8), gamma=1.0)
    bd = dev_blob(blob)
    allv = np.arange(-127, 128, dtype=np.int64)
    for b0 in range(0, allv.size, 64):
        v = allv[b0:b0 + 64]
        M = v.size
        x = np.zeros((M, K), np.float32)
        x[:, e] = 127.0
        x[:, c] = v
        act, got = quantize_act_dev(x, M, K)
        assert np.array_equal(got["q"][:, c], v)
        if fmt == bq.W2A8:
            out = run_gemv(desc, bd, act, bq.DT_ACT, M, bq.F_ACC_INT32, M * ncodes * 2)
            A = out.reshape(M, ncodes, 2)[:, :, c // 128]
            assert np.array_equal(A, np.outer(v, np.arange(ncodes)))
        elif fmt == bq.BVSR4:
            out = run_gemv(desc, bd, act, bq.DT_ACT, M, bq.F_ACC_INT32, M * ncodes * 8 * 4)
            P = out.reshape(M, ncodes, 8, 4)[:, :, c // 32, :]
            bits = (np.arange(ncodes)[:, None] >> np.arange(4)[None, :]) & 1
            assert np.array_equal(P, v[:, None, None] * bits[None])
        else:
            Y = run_gemv(desc, bd, act, bq.DT_ACT, M, bq.F_ACC_INT32, M * ncodes).reshape(M, ncodes)
            assert np.array_equal(Y, np.outer(v, np.arange(ncodes) - 1))


# ====================================================================== HGF
def _hgf_run(desc, blob, xs, M, K, ws=None):
    """bitq_quantize_act_hgf then bitq_gemv/gemm_smallM: returns (act buffer
    on the device, parsed act sections, h [M, r], workspace)."""
    t = torch()
    act_bytes, ws_bytes = bq.hgf_act_size(desc, M)
    act = t.full((act_bytes,), 0x5A, dtype=t.uint8, device="cuda")     # poison
    if ws is None:
        ws = t.zeros(ws_bytes, dtype=t.uint8, device="cuda")
    x = to_dev(xs)
    dt = bq.DT_F32 if xs.dtype == np.float32 else bq.DT_BF16
    bq.quantize_act_hgf(desc, blob, x, dt, M, act, ws)
    t.cuda.synchronize()
    buf = act.cpu().numpy()
    L = bq.act_layout(M, K, desc.rank)
    h = buf[L["off_h"]:L["off_h"] + 4 * M * desc.rank].view(np.float32).reshape(M, desc.rank)
    return act, parse_act(buf, M, K), h.copy(), ws


def _h_tol(xf, A):
    """fp32 bound of the down projection: the run sums (rank terms), the
    256/rank runs and the final rounding give at most 65 2^-24 sum|x A|, times
    max |silu'| < 1.1; exp and the division add a few ulp of |h|."""
    ref = og.lora_down(xf, A)
    zabs = np.abs(np.asarray(xf, np.float64)) @ np.abs(np.asarray(A, np.float64))
    return ref, 1e-5 * zabs + 1e-6 * np.abs(ref) + 1e-30


def _hgf_case(N, K, M, r, W, xs, xf, A, B, alpha, rows=None, T=None):
    q, d = oact.quantize(xf)
    if T is None:
        T, gamma = ow.quantize_ternary(W)
    else:
        gamma = np.float32(0.0125)
    desc = bq.wdesc(bq.HGF, N, K, rank=r)
    blob = bq.pack_weights(desc, tern=T, gamma=gamma, lora_a=A, lora_b=B, lora_alpha=alpha)
    bd = dev_blob(blob)
    act, pa, h, ws = _hgf_run(desc, bd, xs, M, K)
    _act_matches(pa, xf, K)          # the int8 sections are bitq_quantize_act's, bit for bit
    A64, B64 = A.astype(np.float64), B.astype(np.float64)
    h_ref, h_tol = _h_tol(xf, A64)
    assert_within(h, h_ref, h_tol, f"hgf h {N}x{K} r={r} M={M}")
    assert not ws.cpu().numpy().any(), "workspace left non-zero"
    r_ = np.arange(N) if rows is None else rows
    Yi = run_gemv(desc, bd, act, bq.DT_ACT, M, bq.F_ACC_INT32, M * N).reshape(M, N)
    assert np.array_equal(Yi[:, r_], og.ternary_int(T[r_], q)), "hgf Y_int"
    y = run_gemv(desc, bd, act, bq.DT_ACT, M)
    y_ref, tol = og.gemv_hgf(T[r_], gamma, q, d, xf, A64, B64[:, r_], np.float32(alpha))
    assert_within(y[:, r_], y_ref, tol, f"hgf y {N}x{K} r={r} M={M}")
    return desc, bd, act, y, h


def _hgf_inputs(N, K, M, r, shape_idx=0, sigma_ab=0.02, seed=0, f32=False):
    W = synth.gaussian_f32(np.random.default_rng(7 * N + K + seed), (N, K), 0.02)
    if f32:
        xf = synth.gaussian_f32(np.random.default_rng(M + seed), (M, K), 1.0)
        xs = xf
    else:
        xs, xf = synth.random_bf16(np.random.default_rng(M + seed), (M, K))
    Ab, Bb, alpha = synth.lora_params(shape_idx, N, K, r, sigma=sigma_ab, seed_offset=seed)
    return W, xs, xf, Ab.view(np.float16), Bb.view(np.float16), alpha


@pytest.mark.parametrize("N,K,M,r", [(70, 224, 1, 32), (130, 32, 1, 8), (200, 1056, 4, 16), (64, 4096, 1, 64),
                                     (300, 416, 16, 32), (100, 16128, 1, 8), (520, 2048, 64, 64)])
def test_hgf_gemv(N, K, M, r):
    say("hgf", N, K, M, r)
    W, xs, xf, A, B, alpha = _hgf_inputs(N, K, M, r)
    _hgf_case(N, K, M, r, W, xs, xf, A, B, alpha)


def test_hgf_f32_input_and_saturated_silu():
    # A ~ N(0, 1): |z| reaches tens, so silu saturates on both sides
    N, K, M, r = 130, 512, 2, 16
    say("hgf f32 saturated", N, K, M, r)
    W, xs, xf, A, B, alpha = _hgf_inputs(N, K, M, r, sigma_ab=1.0, f32=True)
    _, _, _, _, h = _hgf_case(N, K, M, r, W, xs, xf, A, B, np.float32(-0.8))
    assert (h < -1e-3).any() and (h > 20).any()


def test_hgf_correction_alone_and_zero_b():
    N, K, M, r = 200, 768, 3, 32
    say("hgf isolated paths", N, K, M, r)
    W, xs, xf, A, B, alpha = _hgf_inputs(N, K, M, r, sigma_ab=0.5)
    # T = 0: y is the correction alone, checked with its own (tight) bound
    T0 = np.zeros((N, K), np.int8)
    _, _, _, y, _ = _hgf_case(N, K, M, r, W, xs, xf, A, B, np.float32(1.5), T=T0)
    ref, tol = og.lora_correction(xf, A.astype(np.float64), B.astype(np.float64), np.float32(1.5))
    assert_within(y, ref, tol, "correction alone")
    assert np.abs(ref).max() > 1.0
    # B = 0: the HGF output equals the TERNARY kernel's, bit for bit
    Bz = np.zeros_like(B)
    desc, bd, act, y0, _ = _hgf_case(N, K, M, r, W, xs, xf, A, Bz, alpha)
    T, gamma = ow.quantize_ternary(W)
    dt = bq.wdesc(bq.TERNARY, N, K)
    bt = dev_blob(bq.pack_weights(dt, tern=T, gamma=gamma))
    yt = run_gemv(dt, bt, act, bq.DT_ACT, M)       # the HGF buffer starts with the int8 sections
    assert np.array_equal(y0.view(np.uint32), yt.view(np.uint32))


def test_hgf_zero_token_deterministic_and_workspace_reuse():
    N, K, M, r = 256, 1152, 4, 32
    say("hgf determinism", N, K, M, r)
    W, xs, xf, A, B, alpha = _hgf_inputs(N, K, M, r)
    xs = xs.copy()
    xf = xf.copy()
    xs[2] = 0
    xf[2] = 0.0                                      # an all-zero token: d = 0, h = 0, y = 0
    desc, bd, act, y, h = _hgf_case(N, K, M, r, W, xs, xf, A, B, alpha)
    assert np.all(h[2] == 0) and np.all(y[2] == 0)
    _, _, h2, ws = _hgf_run(desc, bd, xs, M, K)
    for _ in range(3):                               # the same workspace, reused without clearing
        _, _, h3, ws = _hgf_run(desc, bd, xs, M, K, ws=ws)
        assert np.array_equal(h3.view(np.uint32), h.view(np.uint32))
    assert np.array_equal(h2.view(np.uint32), h.view(np.uint32))
    # batch invariance: token m of the batch equals the M = 1 result
    act1, _, h1, _ = _hgf_run(desc, bd, xs[1:2], 1, K)
    assert np.array_equal(h1[0].view(np.uint32), h[1].view(np.uint32))
    y1 = run_gemv(desc, bd, act1, bq.DT_ACT, 1)
    assert np.array_equal(y1[0].view(np.uint32), y[1].view(np.uint32))


@pytest.mark.parametrize("N,K,M,r", [(512, 512, 1, 32), (2048, 512, 1, 32), (512, 2048, 16, 32),
                                     (4096, 4096, 1, 32), (4096, 4096, 16, 64), (11008, 4096, 1, 32)])
def test_hgf_workload(N, K, M, r):
    say("hgf workload", N, K, M, r)
    si = {(512, 512): 0, (2048, 512): 1, (512, 2048): 2, (4096, 4096): 3}.get((N, K), 0)
    W = synth.weights("ternary", si, N, K)
    xs, xf = synth.activations("ternary", si, M, K)
    Ab, Bb, alpha = synth.lora_params(si, N, K, r)
    _hgf_case(N, K, M, r, W, xs, xf, Ab.view(np.float16), Bb.view(np.float16), alpha)


# ====================================== int8 matrix-core small-M kernel (M >= 2)
@pytest.mark.parametrize("M", [2, 17, 33, 50])
@pytest.mark.parametrize("fmt,N,K", [(bq.TERNARY, 70, 224), (bq.TERNARY, 200, 1056), (bq.W2A8, 130, 1152),
                                     (bq.W2A8, 64, 128)])
def test_mfma_ragged(fmt, N, K, M):
    say("mfma ragged", fmt, N, K, M)
    W = synth.gaussian_f32(np.random.default_rng(N * K + M), (N, K), 0.02)
    xs, xf = synth.random_bf16(np.random.default_rng(M + 3), (M, K))
    _int_case(fmt, N, K, M, W, xs, xf)


@pytest.mark.parametrize("fmt,N,K,M", [(bq.W2A8, 12352, 256, 40), (bq.TERNARY, 13000, 384, 64),
                                       (bq.W2A8, 16, 4096, 16), (bq.W2A8, 4160, 1152, 4)])
def test_mfma_row_ranges(fmt, N, K, M):
    # more 16-row sub-tiles than one pass of the 256 workgroups holds (several
    # passes, the last one partial), fewer sub-tiles than workgroups, ragged N
    say("mfma row ranges", fmt, N, K, M)
    W = synth.gaussian_f32(np.random.default_rng(N + K + M), (N, K), 0.02)
    xs, xf = synth.random_bf16(np.random.default_rng(M + 11), (M, K))
    _int_case(fmt, N, K, M, W, xs, xf)


@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("m,M", [(4, 5), (8, 64), (3, 2)])
def test_mfma_wnam(n, m, M):
    N, K = 190, 640
    say("mfma wnam", n, m, M)
    W = synth.gaussian_f32(np.random.default_rng(n * 10 + m), (N, K), 0.02)
    xs, xf = synth.random_bf16(np.random.default_rng(M + n), (M, K))
    _wnam_case(N, K, M, n, m, W, xs, xf)


def test_mfma_extreme_codes_and_activations():
    # all weight codes at the extremes of their range against +-127 (and the
    # most negative sums): the int32 group sums must still be exact
    N, K, M = 64, 512, 20
    say("mfma extremes", N, K, M)
    rng = np.random.default_rng(99)
    for fmt in (bq.W2A8, bq.TERNARY):
        x = np.where(rng.random((M, K)) < 0.5, 127.0, -127.0).astype(np.float32)
        x[:, 0] = 127.0
        x[3] = -127.0
        x[3, 0] = 127.0
        if fmt == bq.W2A8:
            code = np.full((N, K), 3, np.uint8)
            code[::2] = 0
            desc = bq.wdesc(fmt, N, K)
            blob = bq.pack_weights(desc, code=code, delta=np.ones((N, K // 128), np.float16),
                                   zero=np.zeros((N, K // 128), np.float16))
        else:
            code = np.where(rng.random((N, K)) < 0.5, 1, -1).astype(np.int8)
            code[5] = -1
            desc = bq.wdesc(fmt, N, K)
            blob = bq.pack_weights(desc, tern=code, gamma=1.0)
        bd = dev_blob(blob)
        act, got = quantize_act_dev(x, M, K)
        q = got["q"][:, :K].astype(np.int64)
        if fmt == bq.W2A8:
            G = K // 128
            A = run_gemv(desc, bd, act, bq.DT_ACT, M, bq.F_ACC_INT32, M * N * G).reshape(M, N, G)
            ref = np.einsum("nk,mk->mnk", code.astype(np.int64), q).reshape(M, N, G, 128).sum(-1)
        else:
            A = run_gemv(desc, bd, act, bq.DT_ACT, M, bq.F_ACC_INT32, M * N).reshape(M, N)
            ref = q @ code.astype(np.int64).T
        assert np.array_equal(A, ref), fmt


@pytest.mark.parametrize("M", [1, 3, 16, 64])
def test_wnam_bit_balance(M):
    # the symmetric five-level grid on three planes (z = 2), M = 1/3 on the
    # VALU kernel and 16/64 on the matrix cores
    N, K = 11008 if M == 1 else 520, 4096
    say("wnam bit balance", N, K, M)
    W = synth.weights("w2a8", 1, N, K)
    xs, xf = synth.activations("w2a8", 1, M, K)
    rows = np.arange(0, N, 37) if N > 1024 else None
    _wnam_case(N, K, M, 3, 8, W, xs, xf, rows=rows, balanced=True)


# ============================================================ maximum sizes
@pytest.mark.parametrize("fmt", [bq.TERNARY, bq.W2A8])
@pytest.mark.parametrize("M", [1, 4])
def test_max_k_integer(fmt, M):
    # K = 2^20 (the largest the ABI accepts): many rounds of k blocks per
    # workgroup on the VALU kernel, 64+ blocks per wave on the matrix cores
    N, K = 64, 1 << 20
    say("max K", fmt, N, K, M)
    rng = np.random.default_rng(M)
    W = synth.gaussian_f32(rng, (N, K), 0.02)
    xs, xf = synth.random_bf16(rng, (M, K))
    _int_case(fmt, N, K, M, W, xs, xf)


@pytest.mark.parametrize("M", [1, 4, 8])
def test_large_n_integer(M):
    # 2^20 output rows (16384 row tiles): sampled rows against the oracle
    N, K = 1 << 20, 128
    say("large N", N, K, M)
    rng = np.random.default_rng(7 + M)
    W = synth.gaussian_f32(rng, (N, K), 0.02)
    xs, xf = synth.random_bf16(rng, (M, K))
    rows = np.concatenate([np.arange(0, 64), rng.choice(N, 2000, replace=False), np.arange(N - 64, N)])
    _int_case(bq.TERNARY, N, K, M, W, xs, xf, rows=rows)


@pytest.mark.parametrize("M", [1, 3])
def test_max_k_xnor(M):
    N, K = 64, 64512          # the SIGN1 descriptor's largest K
    say("max K xnor", N, K, M)
    xs, xf = synth.random_bf16(np.random.default_rng(11 + M), (M, K))
    _xnor_case(N, K, M, xs, xf, seed=5)
