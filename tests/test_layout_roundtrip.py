"""Host packer (library, C++) -> blob -> independent oracle reader: the logical
form comes back bit for bit, padding is zero, and the header is as specified."""
import numpy as np
import pytest

import bit_plane_gemv_amd as bq
from oracle import layout, weights as ow
import synth

SHAPES = [(64, 128), (70, 224), (1, 32), (130, 416)]


def _w(N, K, sigma=0.02, seed=0):
    return synth.gaussian_f32(np.random.default_rng(seed), (N, K), sigma)


@pytest.mark.parametrize("N,K", SHAPES)
def test_roundtrip_sign(N, K):
    B, alpha = ow.quantize_sign(_w(N, K, 1.0))
    blob = bq.pack_weights(bq.wdesc(bq.SIGN1, N, K), sign=B, alpha=alpha)
    out = layout.unpack(blob)
    h = out["header"]
    assert (h["fmt"], h["N"], h["K"], h["P"], h["version"]) == (1, N, K, 1, 1)
    assert h["total"] == blob.nbytes and h["off_planes"] == 256
    assert np.array_equal(out["B"], B) and np.array_equal(out["alpha"], alpha) and out["pad_ok"]
    assert list(h["hbound"]) == [1.0, 0.0, 0.0]


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("P", [1, 2, 3])
def test_roundtrip_rabit(N, K, P):
    B, g, h = ow.quantize_rabit(_w(N, K), paths=P)
    blob = bq.pack_weights(bq.wdesc(bq.RABIT, N, K, planes=P), sign=B, g=g, h=h)
    out = layout.unpack(blob)
    assert np.array_equal(out["B"], B) and out["pad_ok"]
    assert np.array_equal(out["g"].view(np.uint16), g.view(np.uint16))
    assert np.array_equal(out["h"].view(np.uint16), h.view(np.uint16))
    # header bound of the split-k fixed point: max |h_p| per path, zero past P
    hb = out["header"]["hbound"]
    assert list(hb[:P]) == [float(np.max(np.abs(h[p].astype(np.float64)))) for p in range(P)]
    assert not np.any(hb[P:])


@pytest.mark.parametrize("N,K", SHAPES)
def test_roundtrip_ternary(N, K):
    T, gamma = ow.quantize_ternary(_w(N, K))
    blob = bq.pack_weights(bq.wdesc(bq.TERNARY, N, K), tern=T, gamma=gamma)
    out = layout.unpack(blob)
    assert np.array_equal(out["T"], T) and out["gamma"] == gamma and not out["both_set"]
    assert out["pad_ok"]


@pytest.mark.parametrize("N,K", [(64, 128), (70, 256), (1, 128), (130, 384)])
def test_roundtrip_w2a8(N, K):
    q, delta, zero = ow.quantize_w2a8(_w(N, K))
    blob = bq.pack_weights(bq.wdesc(bq.W2A8, N, K), code=q, delta=delta, zero=zero)
    out = layout.unpack(blob)
    assert np.array_equal(out["q"], q) and out["pad_ok"]
    assert np.array_equal(out["delta"].view(np.uint16), delta.view(np.uint16))
    assert np.array_equal(out["zero"].view(np.uint16), zero.view(np.uint16))


@pytest.mark.parametrize("N,K", SHAPES)
def test_roundtrip_bvsr(N, K):
    rng = np.random.default_rng(N * 1000 + K)
    code = rng.integers(0, 16, (N, K)).astype(np.uint8)
    idx = rng.integers(0, 256, (N, K // 32)).astype(np.uint8)
    cache = rng.standard_normal((256, 5)).astype(np.float32)
    blob = bq.pack_weights(bq.wdesc(bq.BVSR4, N, K), code=code, idx=idx, cache=cache)
    out = layout.unpack(blob)
    assert np.array_equal(out["code"], code) and np.array_equal(out["idx"], idx)
    assert np.array_equal(out["cache"], cache) and out["pad_ok"]


def test_sections_are_256_aligned():
    for fmt in (1, 2, 3, 4, 5):
        blob = np.zeros(0)
        d = bq.wdesc(fmt, 70, 256)
        n = bq.packed_size(d)
        assert n % 256 == 0
        rng = np.random.default_rng(fmt)
        if fmt == 1:
            blob = bq.pack_weights(d, sign=np.ones((70, 256), np.int8), alpha=np.ones(70, np.float32))
        elif fmt == 2:
            blob = bq.pack_weights(d, sign=np.ones((2, 70, 256), np.int8), g=np.ones((2, 70), np.float16),
                                   h=np.ones((2, 256), np.float16))
        elif fmt == 3:
            blob = bq.pack_weights(d, tern=np.zeros((70, 256), np.int8), gamma=1.0)
        elif fmt == 4:
            blob = bq.pack_weights(d, code=np.zeros((70, 256), np.uint8), delta=np.ones((70, 2), np.float16),
                                   zero=np.zeros((70, 2), np.float16))
        else:
            blob = bq.pack_weights(d, code=rng.integers(0, 16, (70, 256)).astype(np.uint8),
                                   idx=np.zeros((70, 8), np.uint8), cache=np.zeros((256, 5), np.float32))
        h = layout.parse_header(blob)
        for k in ("off_planes", "off_c0", "off_c1", "total"):
            assert h[k] % 256 == 0


@pytest.mark.parametrize("N,K", [(64, 128), (130, 384)])
@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_roundtrip_wnam(N, K, n):
    q, delta, zero = ow.quantize_wnam(_w(N, K), n)
    d = bq.wdesc(bq.WNAM, N, K, planes=n, abits=4)
    blob = bq.pack_weights(d, code=q, delta=delta, zero=zero)
    out = layout.unpack(blob)
    assert out["format"] == "wnam" and out["header"]["P"] == n and out["pad_ok"]
    assert np.array_equal(out["q"], q)
    assert np.array_equal(out["delta"].view(np.uint16), delta.view(np.uint16))
    assert np.array_equal(out["zero"].view(np.uint16), zero.view(np.uint16))


@pytest.mark.parametrize("n", [1, 3, 4])
def test_library_wnam_quantizer_matches_oracle(n):
    W = _w(96, 512, seed=5)
    d = bq.wdesc(bq.WNAM, 96, 512, planes=n, abits=6)
    out = layout.unpack(bq.quantize_weights(d, W))
    q, delta, zero = ow.quantize_wnam(W, n)
    assert np.array_equal(out["q"], q)
    assert np.array_equal(out["delta"].view(np.uint16), delta.view(np.uint16))
    assert np.array_equal(out["zero"].view(np.uint16), zero.view(np.uint16))


def _rabit_err(W, B, g, h):
    What = sum(ow.rabit_path(B[p], g[p], h[p]) for p in range(B.shape[0]))
    return float(np.sum((W.astype(np.float64) - What) ** 2))


@pytest.mark.parametrize("sweeps", [0, 5])
def test_library_rabit_quantizer_close_to_oracle(sweeps):
    """Library (C++, threaded power iteration) against the oracle: the power
    iterations add in different orders, so the fp16 scales may differ by an
    ulp and a few near-zero residual signs may flip; the fit is the same."""
    W = _w(64, 256, seed=11)
    d = bq.wdesc(bq.RABIT, 64, 256, planes=2)
    out = layout.unpack(bq.quantize_weights(d, W, svid_sweeps=sweeps))
    B, g, h = ow.quantize_rabit(W, 2, svid_sweeps=sweeps)
    assert np.mean(out["B"] == B) > 0.999
    for a, b in ((out["g"], g), (out["h"], h)):
        a64, b64 = a.astype(np.float64), b.astype(np.float64)
        assert np.all(np.abs(a64 - b64) <= 2.0 ** -9 * np.abs(b64) + 1e-7)
    e_lib, e_orc = _rabit_err(W, out["B"], out["g"], out["h"]), _rabit_err(W, B, g, h)
    assert abs(e_lib - e_orc) <= 1e-3 * e_orc


def test_library_rabit_svid_invariants():
    W = _w(96, 384, seed=12)
    d = bq.wdesc(bq.RABIT, 96, 384, planes=2)
    g0 = layout.unpack(bq.quantize_weights(d, W))
    s20 = layout.unpack(bq.quantize_weights(d, W, svid_sweeps=20))
    # the last path is the sign of what the first leaves, from the stored values
    T = W.astype(np.float64) - ow.rabit_path(s20["B"][0], s20["g"][0], s20["h"][0])
    assert np.array_equal(s20["B"][1], np.where(T >= 0, 1, -1).astype(np.int8))
    assert _rabit_err(W, s20["B"], s20["g"], s20["h"]) < 0.995 * _rabit_err(W, g0["B"], g0["g"], g0["h"])
    assert np.all(s20["g"].astype(np.float64) >= 0) and np.all(s20["h"].astype(np.float64) >= 0)


def test_quantize_options_validation():
    import ctypes
    W = _w(64, 128)
    d = bq.wdesc(bq.RABIT, 64, 128)
    blob = np.zeros(bq.packed_size(d), dtype=np.uint8)
    call = lambda desc, opts: bq._lib.bitq_quantize_weights_opts(ctypes.byref(desc), W.ctypes.data, opts,
                                                                 blob.ctypes.data, blob.nbytes, 1)
    assert call(d, None) == bq.E_ARG
    o = bq.QuantOpts(3)
    o.reserved[2] = 1
    assert call(d, ctypes.byref(o)) == bq.E_ARG
    assert call(d, ctypes.byref(bq.QuantOpts(-1))) == bq.E_ARG
    assert call(bq.wdesc(bq.SIGN1, 64, 128), ctypes.byref(bq.QuantOpts(2))) == bq.E_ARG
    assert call(d, ctypes.byref(bq.QuantOpts(2))) == bq.OK


@pytest.mark.parametrize("N,K,r", [(64, 128, 32), (100, 96, 8), (130, 416, 64), (70, 256, 16)])
def test_roundtrip_hgf(N, K, r):
    W = _w(N, K)
    T, gamma = ow.quantize_ternary(W)
    rng = np.random.default_rng(N + K + r)
    A = rng.normal(0, 0.02, size=(K, r)).astype(np.float16)
    B = rng.normal(0, 0.02, size=(r, N)).astype(np.float16)
    alpha = np.float32(-0.37)
    d = bq.wdesc(bq.HGF, N, K, rank=r)
    blob = bq.pack_weights(d, tern=T, gamma=gamma, lora_a=A, lora_b=B, lora_alpha=alpha)
    u = layout.unpack(blob)
    assert u["format"] == "hgf" and u["pad_ok"] and not u["both_set"]
    np.testing.assert_array_equal(u["T"], T)
    assert u["gamma"] == np.float32(gamma)
    np.testing.assert_array_equal(u["A"].view(np.uint16), A.view(np.uint16))
    np.testing.assert_array_equal(u["B"].view(np.uint16), B.view(np.uint16))
    assert u["alpha"] == alpha and u["header"]["rank"] == r
    # the packer's gate is tanh(alpha) in fp64 rounded to fp32; amax_a = max |A|
    assert u["gate"] == np.float32(np.tanh(np.float64(alpha)))
    assert u["amax_a"] == np.float32(np.abs(A.astype(np.float64)).max())
    # the ternary sections are the TERNARY blob's
    bt = bq.pack_weights(bq.wdesc(bq.TERNARY, N, K), tern=T, gamma=gamma)
    h = u["header"]
    np.testing.assert_array_equal(blob[256:h["off_c1"]], bt[256:h["off_c1"]])


def test_library_hgf_quantizer_matches_oracle():
    N, K, r = 130, 384, 16
    W = _w(N, K)
    Ab, Bb, alpha = synth.lora_params(0, N, K, r)
    d = bq.wdesc(bq.HGF, N, K, rank=r)
    blob = bq.quantize_weights_hgf(d, W, Ab, Bb, alpha)
    T, gamma = ow.quantize_ternary(W)
    ref = bq.pack_weights(d, tern=T, gamma=gamma, lora_a=Ab, lora_b=Bb, lora_alpha=alpha)
    assert np.array_equal(blob, ref)
    with pytest.raises(bq.BitqError):
        bq.quantize_weights_hgf(bq.wdesc(bq.TERNARY, N, K), W, Ab, Bb, alpha)
    bad = Ab.copy()
    bad[0, 0] = 0x7E00                      # NaN
    with pytest.raises(bq.BitqError) as e:
        bq.quantize_weights_hgf(d, W, bad, Bb, alpha)
    assert e.value.status == bq.E_ARG


def test_library_bit_balance_matches_oracle_and_validation():
    import ctypes
    N, K = 130, 512
    W = _w(N, K)
    d = bq.wdesc(bq.WNAM, N, K, planes=3, abits=8)
    blob = bq.quantize_weights(d, W, bit_balance=True)
    c, delta, zero = ow.quantize_bit_balance(W)
    assert np.array_equal(blob, bq.pack_weights(d, code=c, delta=delta, zero=zero))
    u = layout.unpack(blob)
    assert u["q"].max() == 4 and np.all(u["zero"] == 2)
    buf = np.zeros(bq.packed_size(d), dtype=np.uint8)
    call = lambda desc, opts: bq._lib.bitq_quantize_weights_opts(ctypes.byref(desc), W.ctypes.data,
                                                                 ctypes.byref(opts), buf.ctypes.data,
                                                                 buf.nbytes, 1)
    assert call(bq.wdesc(bq.WNAM, N, K, planes=2, abits=8), bq.QuantOpts(0, 1)) == bq.E_ARG
    assert call(bq.wdesc(bq.W2A8, N, K), bq.QuantOpts(0, 1)) == bq.E_ARG
    assert call(d, bq.QuantOpts(0, 2)) == bq.E_ARG
    assert call(d, bq.QuantOpts(0, 1)) == bq.OK
