"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_plane_gemv_amd as bq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    """Every entry point declared in the headers under include/."""
    syms = set()
    inc = os.path.join(ROOT, "include")
    for name in sorted(os.listdir(inc)):
        if name.endswith(".h"):
            text = open(os.path.join(inc, name)).read()
            syms |= set(re.findall(r"^\s*(?:bitq_status|const char\*|int32_t)\s+(bitq_\w+)\s*\(", text, re.M))
    return sorted(syms)


def test_every_declared_symbol_is_exported():
    syms = _declared_symbols()
    assert len(syms) >= 10
    lib = ctypes.CDLL(bq.LIB_PATH)
    for s in syms:
        assert hasattr(lib, s), s
    assert set(syms) == set(bq.EXPORTED)


def test_version_and_error_string():
    assert bq.version() == 1
    with pytest.raises(bq.BitqError):
        bq.packed_size(bq.wdesc(bq.SIGN1, 4, 33))
    assert "multiple of 32" in bq.last_error()


@pytest.mark.parametrize("desc,status", [
    (bq.WDesc(9, 64, 128, 1, 0), bq.E_ARG),
    (bq.WDesc(bq.SIGN1, 0, 128, 1, 0), bq.E_SHAPE),
    (bq.WDesc(bq.SIGN1, 64, 48, 1, 0), bq.E_SHAPE),
    (bq.WDesc(bq.SIGN1, 64, 16, 1, 0), bq.E_SHAPE),
    (bq.WDesc(bq.SIGN1, 64, 128, 2, 0), bq.E_SHAPE),
    (bq.WDesc(bq.RABIT, 64, 128, 4, 0), bq.E_SHAPE),
    (bq.WDesc(bq.TERNARY, 64, 128, 2, 32), bq.E_SHAPE),
    (bq.WDesc(bq.W2A8, 64, 96, 2, 128), bq.E_SHAPE),
    (bq.WDesc(bq.W2A8, 64, 128, 2, 64), bq.E_SHAPE),
    (bq.WDesc(bq.BVSR4, 64, 128, 3, 32), bq.E_SHAPE),
    (bq.WDesc(8, 64, 128, 1, 0), bq.E_ARG),
    (bq.WDesc(bq.HGF, 64, 128, 2, 0, 8, 0), bq.E_SHAPE),        # rank 0
    (bq.WDesc(bq.HGF, 64, 128, 2, 0, 8, 12), bq.E_SHAPE),       # rank not 8/16/32/64
    (bq.WDesc(bq.HGF, 64, 128, 2, 0, 8, 128), bq.E_SHAPE),
    (bq.WDesc(bq.HGF, 64, 16256, 2, 0, 8, 32), bq.E_SHAPE),     # K > 16128
    (bq.WDesc(bq.HGF, 64, 128, 1, 0, 8, 32), bq.E_SHAPE),
    (bq.WDesc(bq.HGF, 64, 128, 2, 0, 4, 32), bq.E_SHAPE),       # int8 activations only
    (bq.WDesc(bq.TERNARY, 64, 128, 2, 0, 8, 32), bq.E_SHAPE),   # rank belongs to HGF
    (bq.WDesc(bq.WNAM, 64, 128, 0, 128, 4), bq.E_SHAPE),
    (bq.WDesc(bq.WNAM, 64, 128, 5, 128, 4), bq.E_SHAPE),
    (bq.WDesc(bq.WNAM, 64, 128, 3, 32, 4), bq.E_SHAPE),
    (bq.WDesc(bq.WNAM, 64, 96, 3, 128, 4), bq.E_SHAPE),
    (bq.WDesc(bq.WNAM, 64, 128, 3, 128, 1), bq.E_SHAPE),
    (bq.WDesc(bq.WNAM, 64, 128, 3, 128, 9), bq.E_SHAPE),
    (bq.WDesc(bq.W2A8, 64, 128, 2, 128, 4), bq.E_SHAPE),
    (bq.WDesc(bq.RABIT, 64, 128, 2, 0, 8), bq.E_SHAPE),
])
def test_descriptor_validation(desc, status):
    with pytest.raises(bq.BitqError) as e:
        bq.packed_size(desc)
    assert e.value.status == status


def test_packed_size_formula():
    # planes + coefficients, each section 256-aligned, plus the 256-byte header
    def a(v):
        return (v + 255) // 256 * 256
    for fmt, N, K, c0, c1 in [
        (bq.SIGN1, 256, 256, 4 * 256, 0),
        (bq.RABIT, 11008, 4096, 2 * 2 * 11008, 2 * 2 * 4096),
        (bq.TERNARY, 512, 2048, 4, 0),
        (bq.W2A8, 4096, 11008, 4 * 4096 * 86, 0),
        (bq.BVSR4, 100, 96, 128 * 4, 5120),
    ]:
        d = bq.wdesc(fmt, N, K)
        Np, Kp = (N + 63) // 64 * 64, (K + 127) // 128 * 128
        planes = Np * Kp * d.planes // 8
        off_c0 = a(256 + planes)
        off_c1 = a(off_c0 + c0)
        assert bq.packed_size(d) == a(off_c1 + c1)
    # HGF: gamma, A^T [r][Kp] and B^T [Np][r] in fp16
    for N, K, r in [(4096, 4096, 32), (100, 96, 8), (2048, 512, 64)]:
        d = bq.wdesc(bq.HGF, N, K, rank=r)
        Np, Kp = (N + 63) // 64 * 64, (K + 127) // 128 * 128
        off_c0 = a(256 + Np * Kp * 2 // 8)
        off_c1 = a(off_c0 + 4)
        off_c2 = a(off_c1 + 2 * r * Kp)
        assert bq.packed_size(d) == a(off_c2 + 2 * Np * r)


def test_pack_rejects_bad_codes_and_capacity():
    d = bq.wdesc(bq.TERNARY, 2, 32)
    T = np.zeros((2, 32), np.int8)
    T[1, 3] = 2
    with pytest.raises(bq.BitqError) as e:
        bq.pack_weights(d, tern=T, gamma=1.0)
    assert e.value.status == bq.E_ARG
    d = bq.wdesc(bq.W2A8, 1, 128)
    with pytest.raises(bq.BitqError) as e:
        bq.pack_weights(d, code=np.full((1, 128), 4, np.uint8), delta=np.ones((1, 1), np.float16),
                        zero=np.zeros((1, 1), np.float16))
    assert e.value.status == bq.E_ARG
    with pytest.raises(bq.BitqError) as e:          # zero point must be an integer 0..3
        bq.pack_weights(d, code=np.zeros((1, 128), np.uint8), delta=np.ones((1, 1), np.float16),
                        zero=np.full((1, 1), 0.5, np.float16))
    assert e.value.status == bq.E_ARG
    d = bq.wdesc(bq.SIGN1, 1, 32)
    lg = bq.Logical()
    B = np.ones((1, 32), np.int8)
    al = np.ones(1, np.float32)
    lg.sign, lg.alpha = B.ctypes.data, al.ctypes.data
    small = np.zeros(16, np.uint8)
    st = bq._lib.bitq_pack_weights(ctypes.byref(d), ctypes.byref(lg), small.ctypes.data, 16)
    assert st == bq.E_CAPACITY
    lg.alpha = None
    big = np.zeros(bq.packed_size(d), np.uint8)
    assert bq._lib.bitq_pack_weights(ctypes.byref(d), ctypes.byref(lg), big.ctypes.data,
                                     big.nbytes) == bq.E_ARG


def test_device_entry_points_validate_before_any_device_call():
    d = bq.wdesc(bq.W2A8, 128, 256)
    ws_need = bq.workspace_size(d, 1)
    good = 1 << 20                              # fake, 256-aligned addresses: never dereferenced
    # null pointer
    assert bq._lib.bitq_gemv(ctypes.byref(d), None, good, bq.DT_ACT, good, good, ws_need, 0, None) == bq.E_ARG
    # raw activations for an integer format
    assert bq._lib.bitq_gemv(ctypes.byref(d), good, good, bq.DT_BF16, good, good, ws_need, 0, None) == bq.E_ARG
    # misaligned blob / activation buffer / workspace
    assert bq._lib.bitq_gemv(ctypes.byref(d), good + 16, good, bq.DT_ACT, good, good, ws_need, 0,
                             None) == bq.E_ALIGN
    assert bq._lib.bitq_gemv(ctypes.byref(d), good, good + 64, bq.DT_ACT, good, good, ws_need, 0,
                             None) == bq.E_ALIGN
    # unknown flag
    assert bq._lib.bitq_gemv(ctypes.byref(d), good, good, bq.DT_ACT, good, good, ws_need, 8,
                             None) == bq.E_ARG
    # integer formats need no workspace; the float formats do
    assert ws_need == 0
    dr = bq.wdesc(bq.RABIT, 4096, 4096)
    wsr = bq.workspace_size(dr, 1)
    assert wsr > 0
    assert bq._lib.bitq_gemv(ctypes.byref(dr), good, good, bq.DT_BF16, good, None, wsr, 0, None) == bq.E_ARG
    assert bq._lib.bitq_gemv(ctypes.byref(dr), good, good, bq.DT_BF16, good, good + 8, wsr, 0,
                             None) == bq.E_ALIGN
    assert bq._lib.bitq_gemv(ctypes.byref(dr), good, good, bq.DT_BF16, good, good, wsr - 1, 0,
                             None) == bq.E_CAPACITY
    # float formats: M = 1 only, raw activations, no integer flag
    ds = bq.wdesc(bq.RABIT, 128, 256)
    wsn = bq.workspace_size(ds, 1)
    assert bq._lib.bitq_gemv(ctypes.byref(ds), good, good, bq.DT_ACT, good, good, wsn, 0, None) == bq.E_ARG
    assert bq._lib.bitq_gemv(ctypes.byref(ds), good, good + 4, bq.DT_BF16, good, good, wsn, 0,
                             None) == bq.E_ALIGN
    assert bq._lib.bitq_gemv(ctypes.byref(ds), good, good, bq.DT_BF16, good, good, wsn, 1,
                             None) == bq.E_UNSUPPORTED
    # small-M range and formats
    assert bq._lib.bitq_gemm_smallM(ctypes.byref(d), good, good, 1, good, good, 1 << 30, 0, None) == bq.E_SHAPE
    assert bq._lib.bitq_gemm_smallM(ctypes.byref(d), good, good, 65, good, good, 1 << 30, 0, None) == bq.E_SHAPE
    assert bq._lib.bitq_gemm_smallM(ctypes.byref(ds), good, good, 4, good, good, 1 << 30, 0,
                                    None) == bq.E_UNSUPPORTED
    # activation quantizer
    n = bq.act_size(4, 256)
    assert bq._lib.bitq_quantize_act(good, bq.DT_BF16, 0, 256, good, n, None) == bq.E_SHAPE
    assert bq._lib.bitq_quantize_act(good, bq.DT_BF16, 4, 100, good, n, None) == bq.E_SHAPE
    assert bq._lib.bitq_quantize_act(good, 7, 4, 256, good, n, None) == bq.E_ARG
    assert bq._lib.bitq_quantize_act(good + 2, bq.DT_BF16, 4, 256, good, n, None) == bq.E_ALIGN
    assert bq._lib.bitq_quantize_act(good, bq.DT_BF16, 4, 256, good, n - 1, None) == bq.E_CAPACITY
    assert bq._lib.bitq_quantize_act_bits(good, bq.DT_BF16, 4, 256, 1, good, n, None) == bq.E_SHAPE
    assert bq._lib.bitq_quantize_act_bits(good, bq.DT_BF16, 4, 256, 9, good, n, None) == bq.E_SHAPE
    # WNAM takes an activation buffer and supports small M
    dw = bq.wdesc(bq.WNAM, 128, 256, planes=3, abits=4)
    assert bq.workspace_size(dw, 1) == 0
    assert bq._lib.bitq_gemv(ctypes.byref(dw), good, good, bq.DT_BF16, good, None, 0, 0, None) == bq.E_ARG
    assert bq._lib.bitq_gemm_smallM(ctypes.byref(dw), good, good, 65, good, None, 0, 0, None) == bq.E_SHAPE


def test_fused_quantizer_flag_validation():
    """BITQ_F_FUSE_QUANT: accepted combinations are checked before any
    device call; the rest return the documented errors."""
    good = 1 << 20
    F = bq.F_FUSE_QUANT
    gemv = bq._lib.bitq_gemv
    d = bq.wdesc(bq.W2A8, 128, 256)
    # raw activations only
    assert gemv(ctypes.byref(d), good, good, bq.DT_ACT, good, None, 0, F, None) == bq.E_ARG
    # 16-byte alignment of x (not the activation buffer's 256)
    assert gemv(ctypes.byref(d), good, good + 8, bq.DT_BF16, good, None, 0, F, None) == bq.E_ALIGN
    assert gemv(ctypes.byref(d), good + 16, good + 16, bq.DT_BF16, good, None, 0, F, None) == bq.E_ALIGN
    # not with the integer-partials flag
    assert gemv(ctypes.byref(d), good, good, bq.DT_BF16, good, None, 0, F | bq.F_ACC_INT32,
                None) == bq.E_UNSUPPORTED
    # K bound of the fused kernel
    dk = bq.wdesc(bq.TERNARY, 64, 16384 + 128)
    assert gemv(ctypes.byref(dk), good, good, bq.DT_F32, good, None, 0, F, None) == bq.E_UNSUPPORTED
    # formats without a fused quantizer
    for fmt, kw in ((bq.RABIT, {}), (bq.SIGN1, {}), (bq.HGF, {"rank": 32})):
        df = bq.wdesc(fmt, 128, 256, **kw)
        assert gemv(ctypes.byref(df), good, good, bq.DT_BF16, good, good, 1 << 20, F, None) == bq.E_UNSUPPORTED
    # small-M entry point: not a fused option
    assert bq._lib.bitq_gemm_smallM(ctypes.byref(d), good, good, 4, good, None, 0, F, None) == bq.E_UNSUPPORTED


def test_act_size_matches_documented_layout():
    for M, K in [(1, 4096), (16, 512), (64, 11008), (3, 96)]:
        assert bq.act_size(M, K) == bq.act_layout(M, K)["total"]


def test_binary_activation_buffer_and_validation():
    for M, K in [(1, 4096), (5, 96), (64, 11008)]:
        assert bq.binact_size(M, K) == bq.binact_layout(M, K)["total"]
    good = 1 << 20
    n = bq.binact_size(2, 256)
    assert bq._lib.bitq_binarize_act(good, bq.DT_BF16, 0, 256, good, n, None) == bq.E_SHAPE
    assert bq._lib.bitq_binarize_act(good, bq.DT_BF16, 2, 100, good, n, None) == bq.E_SHAPE
    assert bq._lib.bitq_binarize_act(good, bq.DT_ACT, 2, 256, good, n, None) == bq.E_ARG
    assert bq._lib.bitq_binarize_act(good, bq.DT_BF16, 2, 256, good + 64, n, None) == bq.E_ALIGN
    assert bq._lib.bitq_binarize_act(good, bq.DT_BF16, 2, 256, good, n - 1, None) == bq.E_CAPACITY
    # binary activations pair with SIGN1 weights only
    dr = bq.wdesc(bq.RABIT, 128, 256)
    assert bq._lib.bitq_gemv(ctypes.byref(dr), good, good, bq.DT_BINARY, good, good, 1 << 20, 0,
                             None) == bq.E_UNSUPPORTED
    ds = bq.wdesc(bq.SIGN1, 128, 256)
    assert bq._lib.bitq_gemv(ctypes.byref(ds), good, good + 16, bq.DT_BINARY, good, None, 0, 0,
                             None) == bq.E_ALIGN
    assert bq._lib.bitq_gemm_smallM(ctypes.byref(ds), good, good, 1, good, None, 0, 0, None) == bq.E_SHAPE
    assert bq._lib.bitq_gemm_smallM(ctypes.byref(dr), good, good, 4, good, None, 0, 0, None) == bq.E_UNSUPPORTED


def _hgf_logical(N, K, r, seed=0):
    rng = np.random.default_rng(seed)
    T = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    A = rng.normal(0, 0.02, size=(K, r)).astype(np.float16)
    B = rng.normal(0, 0.02, size=(r, N)).astype(np.float16)
    return T, A, B


def test_hgf_pack_and_quantize_validation():
    N, K, r = 8, 64, 8
    d = bq.wdesc(bq.HGF, N, K, rank=r)
    T, A, B = _hgf_logical(N, K, r)
    bq.pack_weights(d, tern=T, gamma=0.5, lora_a=A, lora_b=B, lora_alpha=0.1)
    bad = A.copy()
    bad[3, 1] = np.float16(np.inf)
    for kw in (dict(lora_a=bad, lora_b=B, lora_alpha=0.1),
               dict(lora_a=A, lora_b=B, lora_alpha=float("nan"))):
        with pytest.raises(bq.BitqError) as e:
            bq.pack_weights(d, tern=T, gamma=0.5, **kw)
        assert e.value.status == bq.E_ARG
    with pytest.raises(ValueError):                           # lora_b missing: the binding refuses
        bq.pack_weights(d, tern=T, gamma=0.5, lora_a=A, lora_alpha=0.1)
    # ... and so does the C ABI (NULL lora_b), for callers that bypass the binding
    t8 = np.ascontiguousarray(T, dtype=np.int8)
    a16 = np.ascontiguousarray(A.view(np.uint16) if A.dtype == np.float16 else A, dtype=np.uint16)
    lg = bq.Logical()
    lg.tern, lg.gamma, lg.lora_a, lg.lora_alpha = t8.ctypes.data, 0.5, a16.ctypes.data, 0.1
    out = np.zeros(bq.packed_size(d), np.uint8)
    assert bq._lib.bitq_pack_weights(ctypes.byref(d), ctypes.byref(lg), out.ctypes.data, out.nbytes) == bq.E_ARG
    with pytest.raises(bq.BitqError) as e:                    # A, B and alpha are trained inputs
        bq.quantize_weights(d, np.zeros((N, K), np.float32))
    assert e.value.status == bq.E_UNSUPPORTED


def test_hgf_act_size_and_validation():
    d = bq.wdesc(bq.HGF, 128, 256, rank=32)
    for M in (1, 16, 64):
        act, ws = bq.hgf_act_size(d, M)
        lay = bq.act_layout(M, 256, 32)
        assert act == lay["total"] and lay["off_h"] == bq.act_layout(M, 256)["total"]
        assert ws == (8 * M * 32 + 255) // 256 * 256
    with pytest.raises(bq.BitqError):
        bq.hgf_act_size(bq.wdesc(bq.TERNARY, 128, 256), 1)
    with pytest.raises(bq.BitqError):
        bq.hgf_act_size(d, 65)
    good = 1 << 20
    act, ws = bq.hgf_act_size(d, 2)
    f = bq._lib.bitq_quantize_act_hgf
    dt = bq.wdesc(bq.TERNARY, 128, 256)
    assert f(ctypes.byref(dt), good, good, bq.DT_BF16, 2, good, act, good, ws, None) == bq.E_ARG
    assert f(ctypes.byref(d), None, good, bq.DT_BF16, 2, good, act, good, ws, None) == bq.E_ARG
    assert f(ctypes.byref(d), good, good, bq.DT_BF16, 2, good, act, None, ws, None) == bq.E_ARG
    assert f(ctypes.byref(d), good, good, bq.DT_ACT, 2, good, act, good, ws, None) == bq.E_ARG
    assert f(ctypes.byref(d), good, good + 2, bq.DT_BF16, 2, good, act, good, ws, None) == bq.E_ALIGN
    assert f(ctypes.byref(d), good + 16, good, bq.DT_BF16, 2, good, act, good, ws, None) == bq.E_ALIGN
    assert f(ctypes.byref(d), good, good, bq.DT_BF16, 2, good, act, good + 8, ws, None) == bq.E_ALIGN
    assert f(ctypes.byref(d), good, good, bq.DT_BF16, 2, good, act - 1, good, ws, None) == bq.E_CAPACITY
    assert f(ctypes.byref(d), good, good, bq.DT_BF16, 2, good, act, good, ws - 1, None) == bq.E_CAPACITY
    assert f(ctypes.byref(d), good, good, bq.DT_BF16, 0, good, act, good, ws, None) == bq.E_SHAPE
    # the GEMV takes the HGF activation buffer; no workspace
    assert bq.workspace_size(d, 1) == 0
    assert bq._lib.bitq_gemv(ctypes.byref(d), good, good, bq.DT_BF16, good, None, 0, 0, None) == bq.E_ARG


def test_context_kernels_validate_before_any_device_call():
    good = 1 << 20                              # fake, aligned addresses: never dereferenced
    assert bq._lib.bitq_ctx_empty(0, None) == bq.E_SHAPE
    assert bq._lib.bitq_ctx_empty((1 << 20) + 1, None) == bq.E_SHAPE
    assert bq._lib.bitq_ctx_stream(None, 4096, 16, good, 64, None) == bq.E_ARG
    assert bq._lib.bitq_ctx_stream(good, 0, 16, good, 64, None) == bq.E_SHAPE
    assert bq._lib.bitq_ctx_stream(good, 4100, 16, good, 64, None) == bq.E_SHAPE
    assert bq._lib.bitq_ctx_stream(good, 4096, 0, good, 64, None) == bq.E_SHAPE
    assert bq._lib.bitq_ctx_stream(good, 4096, 16, None, 64, None) == bq.E_ARG
    assert bq._lib.bitq_ctx_stream(good, 4096, 16, good, -1, None) == bq.E_SHAPE
    assert bq._lib.bitq_ctx_stream(good + 8, 4096, 16, good, 64, None) == bq.E_ALIGN
    assert bq._lib.bitq_ctx_stream(good, 4096, 16, good + 2, 64, None) == bq.E_ALIGN
    assert bq._lib.bitq_ctx_spin(0, None) == bq.E_SHAPE
    assert bq._lib.bitq_ctx_spin(10001, None) == bq.E_SHAPE


def test_pack_weights_checks_field_shapes():
    d = bq.wdesc(bq.W2A8, 64, 256)
    ok = dict(code=np.zeros((64, 256), np.uint8), delta=np.ones((64, 2), np.float16),
              zero=np.zeros((64, 2), np.float16))
    bq.pack_weights(d, **ok)
    for name, bad in (("code", np.zeros((64, 128), np.uint8)), ("delta", np.ones((64, 1), np.float16)),
                      ("zero", np.zeros((32, 2), np.float16))):
        with pytest.raises(ValueError):
            bq.pack_weights(d, **{**ok, name: bad})
    with pytest.raises(ValueError):
        bq.pack_weights(d, code=ok["code"], delta=ok["delta"])           # zero missing
    dr = bq.wdesc(bq.RABIT, 64, 256, planes=2)
    with pytest.raises(ValueError):                                       # one path of signs for two paths
        bq.pack_weights(dr, sign=np.ones((1, 64, 256), np.int8), g=np.ones((2, 64), np.float16),
                        h=np.ones((2, 256), np.float16))
    db = bq.wdesc(bq.BVSR4, 64, 256)
    with pytest.raises(ValueError):
        bq.pack_weights(db, code=np.zeros((64, 256), np.uint8), idx=np.zeros((64, 8), np.uint8),
                        cache=np.zeros((255, 5), np.float32))
