"""Helpers for the GPU parity tests: run the library through its C ABI on
torch-owned device buffers and read results back as numpy arrays."""
from __future__ import annotations

import sys

import numpy as np

import bit_plane_gemv_amd as bq


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def torch():
    import torch as t
    return t


def to_dev(arr: np.ndarray):
    t = torch()
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return t.from_numpy(a).cuda()


def dev_blob(blob: np.ndarray):
    t = torch()
    d = t.empty(blob.nbytes, dtype=t.uint8, device="cuda")
    d.copy_(t.from_numpy(blob))
    assert d.data_ptr() % 256 == 0
    return d


def workspace(desc, M=1):
    t = torch()
    return t.zeros(bq.workspace_size(desc, M), dtype=t.uint8, device="cuda")


def quantize_act_dev(x_bits_or_f32: np.ndarray, M: int, K: int, abits: int = 8):
    """Run bitq_quantize_act(_bits); returns (device act buffer, parsed host copy)."""
    t = torch()
    x = to_dev(x_bits_or_f32)
    dt = bq.DT_F32 if x_bits_or_f32.dtype == np.float32 else bq.DT_BF16
    act = t.full((bq.act_size(M, K),), 0x5A, dtype=t.uint8, device="cuda")  # poison
    bq.quantize_act(x, dt, M, K, act, abits=abits)
    t.cuda.synchronize()
    return act, parse_act(act.cpu().numpy(), M, K)


def parse_act(buf: np.ndarray, M: int, K: int) -> dict:
    L = bq.act_layout(M, K)
    Kw, Kp = L["Kw"], L["Kp"]
    planes = buf[L["off_planes"]:L["off_planes"] + M * Kw * 32].view(np.uint32).reshape(M, Kw, 8)
    S = buf[L["off_S"]:L["off_S"] + M * Kw * 4].view(np.int32).reshape(M, Kw)
    q = buf[L["off_q"]:L["off_q"] + M * Kp].view(np.int8).reshape(M, Kp)
    T = (M + 15) // 16
    # [b][t][s][g][j][16] -> token m = 16 t + j, block b, word g, half s
    tiles = buf[L["off_qm"]:L["off_qm"] + 16 * T * Kp].view(np.int8).reshape(Kp // 128, T, 2, 4, 16, 16)
    qm = tiles.transpose(1, 4, 0, 3, 2, 5).reshape(16 * T, Kp)[:M]
    d = buf[L["off_d"]:L["off_d"] + 4 * M].view(np.float32)
    amax = buf[L["off_amax"]:L["off_amax"] + 4 * M].view(np.float32)
    return dict(planes=planes, S=S, q=q, qm=qm, d=d, amax=amax, Kw=Kw, Kp=Kp)


# Byte position of input i of a 32-input word in the activation buffer's qm
# section, with the word's two 16-byte halves side by side (include/bitq.h:
# input 8e + 2c + s in half s at byte 4c + e)
QM_POS = np.array([16 * (i & 1) + 4 * ((i >> 1) & 3) + (i >> 3) for i in range(32)])


def qm_from_q(q: np.ndarray) -> np.ndarray:
    """The qm section the header's layout gives for codes q [M, Kp]."""
    M, Kp = q.shape
    out = np.empty_like(q)
    out.reshape(M, Kp // 32, 32)[:, :, QM_POS] = q.reshape(M, Kp // 32, 32)
    return out


def run_gemv(desc, blob_dev, x_dev, x_dtype, M=1, flags=0, out_elems=None, ws=None):
    """bitq_gemv (M = 1) or bitq_gemm_smallM (M > 1); returns a host array
    (fp32 y [M, N], or int32 partials when flags has F_ACC_INT32)."""
    t = torch()
    n = out_elems if out_elems is not None else M * desc.N
    y = t.full((n,), float("nan"), dtype=t.float32, device="cuda")
    ws = workspace(desc, M) if ws is None else ws
    if M == 1:
        bq.gemv(desc, blob_dev, x_dev, x_dtype, y, ws, flags=flags)
    else:
        bq.gemm_smallM(desc, blob_dev, x_dev, M, y, ws, flags=flags)
    t.cuda.synchronize()
    out = y.cpu().numpy()
    if flags & bq.F_ACC_INT32:
        return out.view(np.int32)
    return out.reshape(M, desc.N)


def assert_within(y, y_ref, tol, what=""):
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} outputs outside tolerance; first {tuple(i)}: "
                             f"y={y[tuple(i)]} ref={y_ref[tuple(i)]} tol={tol[tuple(i)]}")
    return float((err / np.maximum(tol, 1e-300)).max())
