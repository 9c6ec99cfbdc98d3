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
