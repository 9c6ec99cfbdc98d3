"""GPU parity of the fused activation quantizer (bitq_gemv with
BITQ_F_FUSE_QUANT: raw x in, the quantizer in the GEMV kernel's prologue).

Bar: y bit-identical to the two-launch path (bitq_quantize_act, then
bitq_gemv on its buffer, whose sections and partial sums the parity tests
check bit for bit against the oracle) wherever both kernels add in the same
order -- ternary layers (exact integer sums: this pins the fused planes and d
at every shape), layers below 4096 rows, and 16384+ rows outside WnAm --, and
within 1 % of the tolerance of it elsewhere (the fused kernel then takes 16
rows per workgroup, the two-launch one 8: another fp32 summation order); and
always within the oracle's tolerance 2e-3 * sum_k |w^ x^| (oracle
quantization of x, oracle GEMV).  Shapes cover
a ragged k tail, 8 and 16 rows per workgroup, 1 to 8 k blocks per lane, the
largest K of the fused path, every WnAm weight-plane count and several
activation bit counts, bf16 and fp32 x, an all-zero token and exact ties.
"""
import numpy as np
import pytest

import bit_plane_gemv_amd as bq
from oracle import act as oact, gemv as og, weights as ow
import synth
from gpuhelp import assert_within, dev_blob, quantize_act_dev, run_gemv, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _random_w2a8_like(rng, N, K, n):
    """Valid n-bit group codes with fp16 scales and integer zero points (the
    GEMV's parity does not depend on how a valid encoding was chosen)."""
    code = rng.integers(0, 1 << n, (N, K), dtype=np.uint8)
    delta = rng.uniform(1e-3, 2e-2, (N, K // 128)).astype(np.float16)
    zero = rng.integers(0, 1 << n, (N, K // 128)).astype(np.float16)
    return code, delta, zero


def _layer(fmt, N, K, seed, n=2, m=8, realistic=True):
    """(desc, device blob, oracle GEMV function of (rows, q, d))."""
    rng = np.random.default_rng(seed)
    if fmt == bq.TERNARY:
        if realistic:
            T, gamma = ow.quantize_ternary(synth.gaussian_f32(rng, (N, K), 0.02))
        else:
            T, gamma = rng.integers(-1, 2, (N, K), dtype=np.int8), np.float32(0.013)
        desc = bq.wdesc(fmt, N, K)
        blob = bq.pack_weights(desc, tern=T, gamma=gamma)
        ref = lambda r, q, d: og.gemv_ternary(T[r], gamma, q, d)  # noqa: E731
    elif fmt in (bq.W2A8, bq.WNAM):
        if realistic:
            W = synth.gaussian_f32(rng, (N, K), 0.02)
            qw, delta, zero = ow.quantize_w2a8(W) if fmt == bq.W2A8 else ow.quantize_wnam(W, n)
        else:
            qw, delta, zero = _random_w2a8_like(rng, N, K, 2 if fmt == bq.W2A8 else n)
        desc = bq.wdesc(fmt, N, K) if fmt == bq.W2A8 else bq.wdesc(fmt, N, K, planes=n, abits=m)
        blob = bq.pack_weights(desc, code=qw, delta=delta, zero=zero)
        ref = lambda r, q, d: og.gemv_w2a8(qw[r], delta[r], zero[r], q, d)  # noqa: E731
    else:
        if realistic:
            W = synth.gaussian_f32(rng, (N, K), 0.015)
            cache = ow.bvsr_cache(W)
            code, idx, _ = ow.bvsr_search(W, cache)
        else:
            cache = ow.bvsr_cache(synth.gaussian_f32(rng, (256, 1024), 0.015))
            code = rng.integers(0, 16, (N, K), dtype=np.uint8)
            idx = rng.integers(0, 256, (N, K // 32), dtype=np.uint8)
        desc = bq.wdesc(fmt, N, K)
        blob = bq.pack_weights(desc, code=code, idx=idx, cache=cache)
        ref = lambda r, q, d: og.gemv_bvsr(code[r], idx[r], cache, q, d)  # noqa: E731
    return desc, dev_blob(blob), ref


def _x(K, seed, dt):
    xs, xf = synth.random_bf16(np.random.default_rng(seed), (1, K))
    if dt == "f32":
        xf = synth.gaussian_f32(np.random.default_rng(seed), (1, K), 1.0)
        xs = xf.copy()
    return xs, xf


def _same_order(desc):
    """Both kernels use the same workgroup shape (so the same fp32 summation
    order), or the sums are exact integers (ternary).  The fused kernel takes
    16 rows per workgroup from 4096 rows on, with 8 waves (32 k-groups) when
    K > 6144; the plain kernel has 4 waves and 8 rows below 16384 rows."""
    if desc.fmt == bq.TERNARY:
        return True
    fused_rg = 16 if desc.N >= 4096 else 8
    plain_rg = 16 if desc.N >= 16384 and desc.fmt != bq.WNAM else 8
    if fused_rg != plain_rg:
        return False
    return fused_rg == 8 or (desc.K + 127) // 128 <= 48


def _check(desc, bd, ref, xs, xf, rows=None):
    """Fused y against the two-launch y (bit for bit where they add in the
    same order) and against the oracle's tolerance."""
    K = desc.K
    m = desc.abits if desc.fmt == bq.WNAM else 8
    dt = bq.DT_F32 if xs.dtype == np.float32 else bq.DT_BF16
    act, _ = quantize_act_dev(xs, 1, K, m)
    y2 = run_gemv(desc, bd, act, bq.DT_ACT)
    y1 = run_gemv(desc, bd, to_dev(xs), dt, flags=bq.F_FUSE_QUANT)
    q, d = oact.quantize(xf, m)
    r = np.arange(desc.N) if rows is None else rows
    y_ref, tol = ref(r, q, d)
    if _same_order(desc):
        same = y1.view(np.uint32) == y2.view(np.uint32)
        assert same.all(), f"fused != two-launch at {np.argwhere(~same)[:4].tolist()}"
    else:
        assert_within(y1[:, r], y2[:, r].astype(np.float64), 0.01 * tol, "fused vs two-launch")
    return assert_within(y1[:, r], y_ref, tol, f"fused fmt {desc.fmt} {desc.N}x{K}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("fmt,N,K", [
    (bq.TERNARY, 1, 32),        # one row, one 32-input word
    (bq.W2A8, 1, 128),          # one row, one group
    (bq.BVSR4, 3, 32),
    (bq.TERNARY, 70, 224),      # ragged k: the last block is partial
    (bq.TERNARY, 4096, 4096),
    (bq.TERNARY, 16448, 512),   # 16 rows per workgroup
    (bq.W2A8, 70, 256),
    (bq.W2A8, 130, 1152),
    (bq.W2A8, 4096, 11008),     # 3 blocks per lane
    (bq.BVSR4, 70, 224),
    (bq.BVSR4, 128, 512),
])
def test_fused_small(fmt, N, K, dt):
    say("fused", fmt, N, K, dt)
    desc, bd, ref = _layer(fmt, N, K, seed=N + K)
    xs, xf = _x(K, N * 3 + K, dt)
    if fmt == bq.W2A8 and K >= 4096:
        rows = np.sort(np.random.default_rng(1).choice(N, 512, replace=False))
    else:
        rows = None
    say("max err/tol", _check(desc, bd, ref, xs, xf, rows))


@pytest.mark.parametrize("n,m", [(1, 8), (2, 4), (3, 3), (4, 2), (4, 4), (3, 6), (2, 8)])
def test_fused_wnam(n, m):
    N, K = 130, 4096
    say("fused wnam", n, m, N, K)
    desc, bd, ref = _layer(bq.WNAM, N, K, seed=n * 10 + m, n=n, m=m)
    xs, xf = synth.activations("w2a8", 0, 1, K)
    _check(desc, bd, ref, xs, xf)


@pytest.mark.parametrize("n,m,N,K", [(3, 6, 4096, 8192), (2, 4, 4100, 16384), (1, 8, 4096, 1024), (4, 3, 5000, 4096)])
def test_fused_wnam_16_rows(n, m, N, K):
    # 4096+ rows: the fused WnAm kernel takes 16 rows per workgroup (1, 4 or
    # 8 blocks per lane here)
    say("fused wnam 16 rows", n, m, N, K)
    desc, bd, ref = _layer(bq.WNAM, N, K, seed=n + m + K, n=n, m=m, realistic=False)
    xs, xf = _x(K, N + K, "bf16")
    rows = np.sort(np.concatenate([np.arange(0, 32), np.arange(N - 32, N),
                                   np.random.default_rng(K).choice(np.arange(32, N - 32), 256, replace=False)]))
    _check(desc, bd, ref, xs, xf, rows)


@pytest.mark.parametrize("fmt,N,K,dt", [
    (bq.W2A8, 11008, 4096, "bf16"),     # the headline layer
    (bq.W2A8, 16400, 16384, "bf16"),    # 16 rows per workgroup, 8 blocks per lane, largest K
    (bq.TERNARY, 130, 16384, "f32"),    # largest K, 4 blocks per lane
    (bq.BVSR4, 28672, 8192, "bf16"),    # the large BVSR layer
    (bq.WNAM, 11008, 4096, "bf16"),     # W4A4
])
def test_fused_workload_shapes(fmt, N, K, dt):
    say("fused workload", fmt, N, K, dt)
    realistic = fmt == bq.W2A8 and N == 11008
    desc, bd, ref = _layer(fmt, N, K, seed=K + 7, n=4, m=4, realistic=realistic)
    if fmt == bq.W2A8 and N == 11008:
        xs, xf = synth.activations("w2a8", 1, 1, K)
    else:
        xs, xf = _x(K, N + 1, dt)
    if N <= 384:
        rows = None
    else:
        rows = np.sort(np.concatenate([np.arange(0, 64), np.arange(N - 64, N),
                                       np.random.default_rng(N).choice(np.arange(64, N - 64), 256, replace=False)]))
    say("max err/tol", _check(desc, bd, ref, xs, xf, rows))


def test_fused_zero_token_and_ties():
    """x = 0 gives d = 0 and y = 0 exactly; x with amax 127 (s = 1) places
    inputs on exact .5 ties (rounded half to even) and on +-amax."""
    N, K = 200, 512
    for fmt in (bq.TERNARY, bq.W2A8, bq.BVSR4):
        desc, bd, ref = _layer(fmt, N, K, seed=fmt)
        say("fused zero token", fmt)
        xz = np.zeros((1, K), np.float32)
        _check(desc, bd, ref, xz, xz)
        y = run_gemv(desc, bd, to_dev(xz), bq.DT_F32, flags=bq.F_FUSE_QUANT)
        assert np.all(y.view(np.uint32) & 0x7FFFFFFF == 0)
        say("fused ties", fmt)
        x = np.zeros((1, K), np.float32)
        ties = np.array([127.0, -127.0, 0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 126.5, -126.5, 63.5, 64.5],
                        np.float32)
        x[0, :ties.size] = ties
        x[0, ties.size:] = np.random.default_rng(3).uniform(-127, 127, K - ties.size).astype(np.float32)
        x[0, 300] = 127.0
        _check(desc, bd, ref, x, x)
