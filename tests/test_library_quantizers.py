"""The library's offline quantizers (C++, bitq_quantize_weights) against the
oracle's (NumPy, oracle/weights.py), on the CPU.  The two are written
independently; the library's blob is read back by the oracle's own blob
reader (oracle/layout.py) and compared with the oracle's logical form.

  SIGN1   [BitNet] §2.1-2.2: signs and the per-row alpha, bit for bit
  W2A8    [ABQ] §3.2 Eq. (3): codes, delta and zero point, bit for bit
          (the W2A8 descriptor and WNAM with 2 planes)
  BVSR4   [BVSR] introduction: the 256-set coefficient cache bit for bit;
          the per-group set index and codes of the exhaustive search equal,
          except where two sets give the same group error to 1e-12
          (relative), where any of them is a correct answer

Planted mistakes in the oracle's cache construction and in its search
objective show that the BVSR comparison can tell a plausible error from the
intended arithmetic.
"""
import numpy as np
import pytest

import bit_plane_gemv_amd as bq
from oracle import layout, weights as ow
import synth


def _w(N, K, sigma, seed):
    return synth.gaussian_f32(np.random.default_rng(seed), (N, K), sigma)


@pytest.mark.parametrize("N,K,seed", [(96, 512, 1), (130, 416, 2), (1, 32, 3), (257, 4096, 4)])
def test_library_sign_quantizer_matches_oracle(N, K, seed):
    W = _w(N, K, 1.0, seed)
    W[0, :4] = [0.0, -0.0, 1.5, -2.0]            # the tie at zero goes to +1, also for -0.0
    out = layout.unpack(bq.quantize_weights(bq.wdesc(bq.SIGN1, N, K), W))
    B, alpha = ow.quantize_sign(W)
    assert np.array_equal(out["B"], B)
    assert np.array_equal(out["alpha"].view(np.uint32), alpha.view(np.uint32))


@pytest.mark.parametrize("N,K,seed", [(96, 512, 5), (130, 384, 6), (1, 128, 7), (257, 4096, 8)])
@pytest.mark.parametrize("fmt", ["w2a8", "wnam2"])
def test_library_w2a8_quantizer_matches_oracle(N, K, seed, fmt):
    W = _w(N, K, 0.02, seed)
    W[0, :128] = 0.0                              # a flat group: delta := 1, z := 0, q := 0
    d = bq.wdesc(bq.W2A8, N, K) if fmt == "w2a8" else bq.wdesc(bq.WNAM, N, K, planes=2, abits=8)
    out = layout.unpack(bq.quantize_weights(d, W))
    q, delta, zero = ow.quantize_w2a8(W) if fmt == "w2a8" else ow.quantize_wnam(W, 2)
    assert np.array_equal(out["q"], q)
    assert np.array_equal(out["delta"].view(np.uint16), delta.view(np.uint16))
    assert np.array_equal(out["zero"].view(np.uint16), zero.view(np.uint16))
    assert out["q"][0, :128].max() == 0 and float(out["delta"][0, 0]) == 1.0


def _bvsr_compare(W, lib, cache, code, idx, sse, max_tie_frac=0.01):
    """Library (lib: the unpacked blob) against the oracle's cache and search.
    Returns the number of groups decided by an SSE tie."""
    N, K = W.shape
    assert np.array_equal(lib["cache"].view(np.uint32), cache.view(np.uint32)), "cache differs"
    same = lib["idx"] == idx
    # groups where the library picked another set: that set must reach the
    # same least error (an exact tie up to 1e-12 relative)
    lcode, lsse = ow.bvsr_encode(W, cache, lib["idx"])
    tie = ~same
    assert np.all(np.abs(lsse[tie] - sse[tie]) <= 1e-12 * np.maximum(sse[tie], 1e-300)), "set not optimal"
    # codes: equal where the index is equal; elsewhere the nearest points of the chosen set
    G = K // 32
    cg, lg = code.reshape(N, G, 32), lib["code"].reshape(N, G, 32)
    assert np.array_equal(cg[same], lg[same]), "codes differ"
    assert np.array_equal(lcode.reshape(N, G, 32)[tie], lg[tie]), "codes not nearest points"
    assert tie.sum() <= max_tie_frac * idx.size, "too many groups differ"
    return int(tie.sum())


@pytest.mark.slow
@pytest.mark.parametrize("N,K,seed", [(128, 1024, 9), (96, 352, 10)])
def test_library_bvsr_quantizer_matches_oracle(N, K, seed):
    W = _w(N, K, 0.015, seed)
    lib = layout.unpack(bq.quantize_weights(bq.wdesc(bq.BVSR4, N, K), W))
    cache = ow.bvsr_cache(W)
    code, idx, sse = ow.bvsr_search(W, cache)
    _bvsr_compare(W, lib, cache, code, idx, sse)


def test_library_bvsr_quantizer_degenerate_groups():
    # repeated groups (identical weights give identical decisions) and a flat
    # tensor region, whose range quantiles are zero
    N, K = 16, 256
    W = _w(N, K, 0.015, 11)
    W[4:8] = W[0:4]
    W[8:10, :64] = 0.0
    lib = layout.unpack(bq.quantize_weights(bq.wdesc(bq.BVSR4, N, K), W))
    cache = ow.bvsr_cache(W)
    code, idx, sse = ow.bvsr_search(W, cache)
    _bvsr_compare(W, lib, cache, code, idx, sse)
    assert np.array_equal(lib["idx"][4:8], lib["idx"][0:4])


def test_planted_mistake_bvsr_cache_is_detected(monkeypatch):
    """A plausible slip in the oracle's cache (quantile levels j/16 instead of
    (j + 1/2)/16) must make the library comparison fail."""
    N, K = 32, 256
    W = _w(N, K, 0.015, 12)
    lib = layout.unpack(bq.quantize_weights(bq.wdesc(bq.BVSR4, N, K), W))
    real_q = ow.quantile_linear
    monkeypatch.setattr(ow, "quantile_linear", lambda s, qf: real_q(s, qf - 0.5 / 16))
    cache = ow.bvsr_cache(W)
    code, idx, sse = ow.bvsr_search(W, cache)
    with pytest.raises(AssertionError):
        _bvsr_compare(W, lib, cache, code, idx, sse)


def test_planted_mistake_bvsr_search_objective_is_detected(monkeypatch):
    """A search that minimizes the total absolute error instead of the squared
    error (a plausible slip) must make the library comparison fail."""
    N, K = 32, 256
    W = _w(N, K, 0.015, 13)
    lib = layout.unpack(bq.quantize_weights(bq.wdesc(bq.BVSR4, N, K), W))

    def search_abs(Wm, cache, chunk=2048):
        Wm = np.asarray(Wm, dtype=np.float32)
        n, k = Wm.shape
        pts = ow.bvsr_points(cache)
        w = Wm.reshape(-1, 32).astype(np.float64)
        best = np.full(w.shape[0], np.inf)
        bid = np.zeros(w.shape[0], np.int64)
        bcode = np.zeros(w.shape, np.int64)
        for s_ in range(pts.shape[0]):
            d = np.abs(w[:, :, None] - pts[s_][None, None, :])
            c = np.argmin(d, axis=-1)
            e = np.take_along_axis(d, c[..., None], axis=-1)[..., 0].sum(axis=1)
            better = e < best
            best[better], bid[better], bcode[better] = e[better], s_, c[better]
        return (bcode.reshape(n, k).astype(np.uint8), bid.reshape(n, k // 32).astype(np.uint8),
                best.reshape(n, k // 32))
    monkeypatch.setattr(ow, "bvsr_search", search_abs)
    cache = ow.bvsr_cache(W)
    code, idx, sse = ow.bvsr_search(W, cache)
    with pytest.raises(AssertionError):
        _bvsr_compare(W, lib, cache, code, idx, sse)
