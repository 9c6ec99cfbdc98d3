"""bitq_quantize_act_hgf_noalloc (the HGF activation step without a workspace
argument: the library's static device scratch holds the down projection's
fixed-point words) against bitq_quantize_act_hgf with a caller workspace.

Both run the same kernel with the same arithmetic, so every section of the
activation buffer (planes, group sums, q, d and h) must be the same bits.
Two calls in a row on the same device, the second with a smaller input
(fewer tokens, shorter K, lower rank): the scratch keeps the last call's
contents, and a call must not depend on them.  h is also checked against the
oracle's down projection within its fp32 bound, and the int8 sections
against the oracle's quantizer, bit for bit.
"""
import numpy as np
import pytest

import bit_plane_gemv_amd as bq
from oracle import act as oact, gemv as og, weights as ow
import synth
from gpuhelp import dev_blob, parse_act, say, to_dev, torch

pytestmark = pytest.mark.gpu


def _inputs(N, K, M, r, seed):
    W = synth.gaussian_f32(np.random.default_rng(100 + seed), (N, K), 0.02)
    xs, xf = synth.random_bf16(np.random.default_rng(200 + seed), (M, K))
    Ab, Bb, alpha = synth.lora_params(0, N, K, r, seed_offset=seed)
    return W, xs, xf, Ab.view(np.float16), Bb.view(np.float16), alpha


def _act_sections(buf, M, K, r):
    L = bq.act_layout(M, K, r)
    out = parse_act(buf, M, K)
    out["h"] = buf[L["off_h"]:L["off_h"] + 4 * M * r].view(np.float32).reshape(M, r)
    return out


@pytest.mark.parametrize("cases", [[(256, 1024, 16, 32), (96, 512, 3, 16)],
                                   [(130, 4096, 64, 64), (64, 256, 1, 8)]])
def test_noalloc_hgf_matches_workspace_entry_point(cases):
    t = torch()
    for i, (N, K, M, r) in enumerate(cases):
        say("hgf noalloc", N, K, M, r, "call", i)
        W, xs, xf, A, B, alpha = _inputs(N, K, M, r, i)
        T, gamma = ow.quantize_ternary(W)
        desc = bq.wdesc(bq.HGF, N, K, rank=r)
        bd = dev_blob(bq.pack_weights(desc, tern=T, gamma=gamma, lora_a=A, lora_b=B, lora_alpha=alpha))
        x = to_dev(xs)
        act_bytes, ws_bytes = bq.hgf_act_size(desc, M)
        act_ws = t.full((act_bytes,), 0x5A, dtype=t.uint8, device="cuda")     # poison
        act_na = t.full((act_bytes,), 0x3C, dtype=t.uint8, device="cuda")
        ws = t.zeros(ws_bytes, dtype=t.uint8, device="cuda")
        bq.quantize_act_hgf(desc, bd, x, bq.DT_BF16, M, act_ws, ws)
        bq.quantize_act_hgf_noalloc(desc, bd, x, bq.DT_BF16, M, act_na)
        t.cuda.synchronize()
        a = _act_sections(act_ws.cpu().numpy(), M, K, r)
        b = _act_sections(act_na.cpu().numpy(), M, K, r)
        for key in ("planes", "S", "q", "d", "h"):
            assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), f"call {i}: {key} differs"
        q, d = oact.quantize(xf)
        assert np.array_equal(b["q"][:, :K], q) and np.array_equal(b["d"].view(np.uint32), d.view(np.uint32))
        ref = og.lora_down(xf, A.astype(np.float64))
        bound = 1e-5 * (np.abs(xf.astype(np.float64)) @ np.abs(A.astype(np.float64))) + 1e-6 * np.abs(ref) + 1e-30
        assert np.all(np.abs(b["h"].astype(np.float64) - ref) <= bound), f"call {i}: h against the oracle"
        assert not ws.cpu().numpy().any()


def test_noalloc_rejects_oversized_and_bad_arguments():
    t = torch()
    d = bq.wdesc(bq.HGF, 64, 256, rank=64)
    act = t.zeros(bq.hgf_act_size(d, 64)[0], dtype=t.uint8, device="cuda")
    x = t.zeros(64 * 256, dtype=t.int16, device="cuda")
    w = t.zeros(bq.packed_size(d), dtype=t.uint8, device="cuda")
    with pytest.raises(bq.BitqError) as e:
        bq.quantize_act_hgf_noalloc(d, w, x, bq.DT_BF16, 65, act)         # M beyond 64
    assert e.value.status == bq.E_SHAPE
    with pytest.raises(bq.BitqError) as e:
        bq.quantize_act_hgf_noalloc(d, w, x, bq.DT_BF16, 64, act, act_bytes=act.numel() - 1)
    assert e.value.status == bq.E_CAPACITY
    with pytest.raises(bq.BitqError) as e:
        bq.quantize_act_hgf_noalloc(d, w, x, bq.DT_ACT, 64, act)
    assert e.value.status == bq.E_ARG
