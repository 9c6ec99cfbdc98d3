#!/usr/bin/env python3
"""Benchmark of the bit-plane GEMV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one batch-1 GEMV y = W^ x over one Llama-2-7B gate/up layer
(11008 x 4096): the RaBiT 2-path residual-binary layer by default (the
workload the headline metric is quoted on), or the W2A8 bit-plane layer
(activation quantizer + AND+popcount GEMV) with --workload w2a8; the other
workloads are listed in WORKLOADS.  --tokens M (integer formats, 2..64) runs
the small-M path instead: M tokens per step, each weight read once, and the
roofline is then the contraction's (int8 matrix cores from 4 tokens on,
else VALU lane-operations).

Measurement:
  * The packed layer is replicated into >= 1 GiB of distinct device copies and
    step i reads copy i mod C, so every step streams its weights from HBM
    (the 256 MB Infinity Cache and the L2s cannot hold the rotation).
  * Inputs are resident in HBM before timing starts.  The K timed steps are
    captured once into a HIP graph and replayed, so host launch overhead is
    not part of the measurement; HIP events recorded on the launch stream
    bracket the replay.
  * value = packed weight bytes x K / elapsed (GB/s); roofline.achieved is the
    same algorithmic byte count divided by the per-launch time of the GEMV
    kernel measured the same way (equal to ms_per_step when the step is that
    single kernel).
  * cpu_baseline: the CPU oracle (explicit fp64 dequantization + dot product)
    on the same layer, timed on the host for a bounded number of repetitions.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
INT8_MFMA_PEAK_TOPS = 5000.0      # MI355X dense int8 matrix-core peak
# VALU lane-operations per second: 256 CUs x 4 SIMDs x 16 lanes per clock x
# 2.4 GHz (one 64-lane instruction every 4 clocks per SIMD)
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
MFMA_MIN_TOKENS = 4               # the library's switch to the matrix-core kernel
ROTATE_BYTES = 1 << 30
KERNEL_SRC = os.path.join(ROOT, "bit_plane_gemv_amd", "csrc", "bitq_kernels.hip")

# HBM bytes moved per launch of the GEMV kernel, from rocprofv3 counter runs
# (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0; factors calibrated on a plain copy
# kernel of known size; profiles/ holds the runs).  Each entry is valid only
# for the kernel source it was measured on (first 16 hex digits of the
# sha256 of bitq_kernels.hip); otherwise traffic is reported as null.
MEASURED_TRAFFIC = {
    "rabit": {"kernels_sha256_16": "bdb103df4f0f03f2", "bytes_per_launch": 13451264},
    "w2a8": {"kernels_sha256_16": "bdb103df4f0f03f2", "bytes_per_launch": 12829696},
    "w2a8+fuse": {"kernels_sha256_16": "bdb103df4f0f03f2", "bytes_per_launch": 12880896},
}


def kernels_sha() -> str:
    import hashlib
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]

# Algorithmic packed bytes of one layer (planes + coefficients), by format.
# HGF: the ternary planes and gamma, A (read by the activation step) and B
# (read by the GEMV), r fp16 per input and per output.
def packed_bytes(fmt: str, N: int, K: int, planes: int = 2, rank: int = 0) -> int:
    if fmt == "hgf":
        return 2 * N * K // 8 + 4 + 2 * rank * K + 2 * rank * N
    if fmt == "wnam":
        return planes * N * K // 8 + 4 * N * (K // 128)
    if fmt == "rabit":
        return 2 * N * K // 8 + 2 * 2 * N + 2 * 2 * K
    if fmt == "w2a8":
        return 2 * N * K // 8 + 4 * N * (K // 128)
    if fmt == "ternary":
        return 2 * N * K // 8 + 4
    if fmt == "bvsr":
        return 4 * N * K // 8 + N * K // 32 + 256 * 5 * 4
    if fmt == "sign":
        return N * K // 8 + 4 * N
    raise ValueError(fmt)


WORKLOADS = {
    "rabit": dict(fmt="rabit", shape_idx=1, N=11008, K=4096),
    "w2a8": dict(fmt="w2a8", shape_idx=1, N=11008, K=4096),
    "rabit_down": dict(fmt="rabit", shape_idx=2, N=4096, K=11008),
    "w2a8_down": dict(fmt="w2a8", shape_idx=2, N=4096, K=11008),
    "bvsr": dict(fmt="bvsr", shape_idx=1, N=28672, K=8192),
    "ternary": dict(fmt="ternary", shape_idx=3, N=4096, K=4096),
    # arbitrary-bit WnAm on the W2A8 layer's data (n weight planes, m-bit activations)
    "w4a4": dict(fmt="wnam", planes=4, abits=4, data="w2a8", shape_idx=1, N=11008, K=4096),
    "w2a4": dict(fmt="wnam", planes=2, abits=4, data="w2a8", shape_idx=1, N=11008, K=4096),
    "w3a8": dict(fmt="wnam", planes=3, abits=8, data="w2a8", shape_idx=1, N=11008, K=4096),
    # ABQ bit balance: the symmetric five-level 2-bit grid on three planes
    "wbb": dict(fmt="wnam", planes=3, abits=8, bit_balance=True, data="w2a8", shape_idx=1, N=11008, K=4096),
    # fully binary XNOR+popcount: SIGN1 weights x sign activations (binarizer + GEMV per step)
    "xnor": dict(fmt="sign", binary=True, data="sign", shape_idx=0, N=11008, K=4096),
    # HGF: ternary layer + rank-32 gated correction (activation step with the
    # down projection, then the fused GEMV); the C3 4096 x 4096 layer, and the
    # headline shape
    "hgf": dict(fmt="hgf", data="ternary", shape_idx=3, N=4096, K=4096, rank=32),
    "hgf_11008": dict(fmt="hgf", data="ternary", shape_idx=4, N=11008, K=4096, rank=32),
}


def kernel_bytes(wl: dict) -> int:
    """Algorithmic bytes the GEMV kernel itself reads per launch (the HGF
    down-projection matrix A is read by the activation step instead)."""
    fmt, N, K = wl["fmt"], wl["N"], wl["K"]
    if fmt == "hgf":
        return 2 * N * K // 8 + 4 + 2 * wl["rank"] * N
    return packed_bytes(fmt, N, K, wl.get("planes", 2))


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def cpu_baseline(wl: dict, budget_s: float = 12.0) -> dict:
    """The oracle as it stands, timed on the host: explicit fp64 dequantization
    and dot product for one GEMV of the workload layer, repeated until about
    `budget_s` seconds of CPU work (at least once)."""
    from oracle import act as oact, gemv as og, layout, weights as ow
    import synth
    fmt, N, K, si = wl["fmt"], wl["N"], wl["K"], wl["shape_idx"]
    data = wl.get("data", fmt)
    W = synth.weights(data, si, N, K)
    xs, xf = synth.activations(data, si, 1, K)
    if fmt == "rabit":
        # the GEMV step only: the logical form is built once, outside the timing
        B, g, h = ow.quantize_rabit(W)
        run = lambda: og.gemv_rabit(B, g, h, xf)
        what = "oracle gemv_rabit (fp64 dequant + dot)"
    elif fmt == "w2a8":
        qw, delta, zero = ow.quantize_w2a8(W)
        def run():
            q, d = oact.quantize(xf)
            return og.gemv_w2a8(qw, delta, zero, q, d)
        what = "oracle act quantize + gemv_w2a8 (fp64 dequant + dot)"
    elif fmt == "wnam":
        if wl.get("bit_balance"):
            qw, delta, zero = ow.quantize_bit_balance(W)
        else:
            qw, delta, zero = ow.quantize_wnam(W, wl["planes"])
        def run():
            q, d = oact.quantize(xf, wl["abits"])
            return og.gemv_w2a8(qw, delta, zero, q, d)
        what = f"oracle {wl['abits']}-bit act quantize + W{wl['planes']} gemv (fp64 dequant + dot)"
    elif fmt == "sign" and wl.get("binary"):
        B, alpha = ow.quantize_sign(W)
        def run():
            xb, beta = oact.binarize(xf)
            return og.gemv_xnor(B, alpha, xb, beta)
        what = "oracle binarize + gemv_xnor (fp64 dequant + dot)"
    elif fmt == "ternary":
        T, gamma = ow.quantize_ternary(W)
        def run():
            q, d = oact.quantize(xf)
            return og.gemv_ternary(T, gamma, q, d)
        what = "oracle act quantize + gemv_ternary (fp64 dequant + dot)"
    elif fmt == "hgf":
        T, gamma = ow.quantize_ternary(W)
        Ab, Bb, alpha = synth.lora_params(si, N, K, wl["rank"])
        A = Ab.view(np.float16).astype(np.float64)
        B = Bb.view(np.float16).astype(np.float64)
        def run():
            q, d = oact.quantize(xf)
            return og.gemv_hgf(T, gamma, q, d, xf, A, B, alpha)
        what = "oracle act quantize + gemv_hgf (fp64 ternary dequant + dot, fp64 correction)"
    elif fmt == "bvsr":
        # logical form from the library's quantizer (the oracle's exhaustive
        # search is far too slow at this size), read back by the oracle
        import bit_plane_gemv_amd as bq
        L = layout.unpack(bq.quantize_weights(bq.wdesc("bvsr", N, K), W))
        def run():
            q, d = oact.quantize(xf)
            return og.gemv_bvsr(L["code"], L["idx"], L["cache"], q, d)
        what = "oracle act quantize + gemv_bvsr (fp64 dequant + dot)"
    else:
        raise ValueError(fmt)
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    times = []
    t_all = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        run()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all > budget_s or len(times) >= 50:
            break
    med = float(np.median(times))
    return {"value": packed_bytes(fmt, N, K, wl.get("planes", 2), wl.get("rank", 0)) / med / 1e9, "unit": "GB/s",
            "cores": int(threads),
            "kind": "oracle",
            "sample": f"{what}, {fmt} {N}x{K} M=1, {len(times)} runs, median {med * 1e3:.1f} ms "
                      f"per GEMV; host has {os.cpu_count()} cpus"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="rabit", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch every step from the host")
    ap.add_argument("--tokens", type=int, default=1,
                    help="tokens per step (integer formats: 2..64 run the small-M path)")
    ap.add_argument("--fuse", action="store_true",
                    help="integer formats, one token: the activation quantizer runs inside the GEMV "
                         "kernel (BITQ_F_FUSE_QUANT), one launch per step")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_plane_gemv_amd as bq
    import synth

    wl = WORKLOADS[args.workload]
    fmt, N, K, si = wl["fmt"], wl["N"], wl["K"], wl["shape_idx"]
    M = args.tokens
    if M != 1 and (fmt in ("rabit",) or (fmt == "sign" and not wl.get("binary")) or not 1 <= M <= 64):
        print("--tokens > 1 needs an integer-activation workload and at most 64 tokens", file=sys.stderr)
        sys.exit(2)
    fuse = args.fuse
    if fuse and (M != 1 or fmt not in ("ternary", "w2a8", "bvsr", "wnam") or wl.get("binary")):
        print("--fuse needs one token and a TERNARY/W2A8/BVSR4/WNAM workload", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- weights: library quantizer + packer (offline, untimed)
    t0 = time.perf_counter()
    data = wl.get("data", fmt)
    W = synth.weights(data, si, N, K)
    desc = bq.wdesc(fmt, N, K, planes=wl.get("planes"), abits=wl.get("abits"), rank=wl.get("rank"))
    abits = wl.get("abits", 8)
    hgf = fmt == "hgf"
    if hgf:
        Ab, Bb, alpha = synth.lora_params(si, N, K, wl["rank"])
        blob = bq.quantize_weights_hgf(desc, W, Ab, Bb, alpha)
    else:
        blob = bq.quantize_weights(desc, W, bit_balance=bool(wl.get("bit_balance")))
    log(f"quantized+packed {fmt} {N}x{K} in {time.perf_counter() - t0:.1f}s, blob {blob.nbytes} B")
    alg_bytes = packed_bytes(fmt, N, K, wl.get("planes", 2), wl.get("rank", 0))
    gemv_bytes = kernel_bytes(wl)
    copies = max(2, math.ceil(ROTATE_BYTES / blob.nbytes))
    base = torch.empty(blob.nbytes, dtype=torch.uint8, device=dev)
    base.copy_(torch.from_numpy(blob))
    stride = (blob.nbytes + 4095) // 4096 * 4096
    pool = torch.empty(copies * stride, dtype=torch.uint8, device=dev)
    for c in range(copies):
        pool[c * stride:c * stride + blob.nbytes].copy_(base)
    del base
    blobs = [pool[c * stride:c * stride + blob.nbytes] for c in range(copies)]

    # ---- activations / outputs / workspace
    xs, xf = synth.activations(data, si, M, K)
    if xs.dtype == np.float32:      # fp32 activations (the sign workloads' inputs)
        x, x_dt = torch.from_numpy(np.ascontiguousarray(xs)).to(dev), bq.DT_F32
    else:                           # bf16 bit patterns
        x, x_dt = torch.from_numpy(np.ascontiguousarray(xs).view(np.int16)).to(dev), bq.DT_BF16
    y = torch.empty(M * N, dtype=torch.float32, device=dev)
    ws = torch.zeros(bq.workspace_size(desc, M), dtype=torch.uint8, device=dev)
    binary = bool(wl.get("binary"))
    integer = fmt in ("ternary", "w2a8", "bvsr", "wnam", "hgf") or binary
    if binary:
        act = torch.zeros(bq.binact_size(M, K), dtype=torch.uint8, device=dev)
    elif hgf:
        act_bytes, act_ws_bytes = bq.hgf_act_size(desc, M)
        act = torch.zeros(act_bytes, dtype=torch.uint8, device=dev)
        act_ws = torch.zeros(act_ws_bytes, dtype=torch.uint8, device=dev)
    else:
        act = torch.zeros(bq.act_size(M, K), dtype=torch.uint8, device=dev) if integer else None
    act_dt = bq.DT_BINARY if binary else bq.DT_ACT
    stream = torch.cuda.current_stream()

    def product(w, a, a_dt, ws_, st):
        """The GEMV (one token) or the small-M GEMM (M tokens)."""
        if M == 1:
            bq.gemv(desc, w, a, a_dt, y, ws_, stream=st)
        else:
            bq.gemm_smallM(desc, w, a, M, y, ws_, stream=st)

    def step(i):
        w = blobs[i % copies]
        if binary:
            bq.binarize_act(x, x_dt, M, K, act, stream=stream)
            product(w, act, bq.DT_BINARY, None, stream)
        elif hgf:
            bq.quantize_act_hgf(desc, w, x, x_dt, M, act, act_ws, stream=stream)
            product(w, act, bq.DT_ACT, None, stream)
        elif fuse:
            bq.gemv(desc, w, x, x_dt, y, None, flags=bq.F_FUSE_QUANT, stream=stream)
        elif integer:
            bq.quantize_act(x, x_dt, M, K, act, stream=stream, abits=abits)
            product(w, act, bq.DT_ACT, ws, stream)
        else:
            bq.gemv(desc, w, x, x_dt, y, ws, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K_steps = args.steps
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                stream = torch.cuda.current_stream()
                for i in range(K_steps):
                    step(i)
        torch.cuda.current_stream().wait_stream(s)
        stream = torch.cuda.current_stream()
        graph.replay()                      # one untimed replay
        torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(K_steps):
            step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / K_steps
    value = alg_bytes / (ms_per_step * 1e-3) / 1e9

    # per-launch time of the GEMV kernel alone (integer workloads also run the
    # activation quantizer in each step): a graph of GEMV launches only
    gemv_ms = ms_per_step
    if integer and graph is not None and not fuse:
        g2 = torch.cuda.CUDAGraph()
        s2 = torch.cuda.Stream()
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s2):
            with torch.cuda.graph(g2, stream=s2):
                st2 = torch.cuda.current_stream()
                for i in range(K_steps):
                    product(blobs[i % copies], act, act_dt, None if binary else ws, st2)
        torch.cuda.current_stream().wait_stream(s2)
        g2.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(torch.cuda.current_stream())
        g2.replay()
        e1.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        gemv_ms = e0.elapsed_time(e1) / K_steps
    achieved = gemv_bytes / (gemv_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4)}
    mfma = M >= MFMA_MIN_TOKENS and fmt in ("ternary", "w2a8", "wnam")
    if M > 1:
        # the small-M contraction: int8 ops (2 M N K) on the matrix cores, or,
        # on the VALU, the AND and popcount lane-operations of the bit planes
        # (2 per weight plane x activation plane x 32 weights x token)
        if mfma:
            tops = 2.0 * M * N * K / (gemv_ms * 1e-3) / 1e12
            roof = {"bound": "mfma", "achieved": round(tops, 2), "peak": INT8_MFMA_PEAK_TOPS, "unit": "TOP/s",
                    "frac": round(tops / INT8_MFMA_PEAK_TOPS, 4)}
        else:
            wplanes = {"ternary": 2, "w2a8": 2, "bvsr": 4, "hgf": 2}.get(fmt, wl.get("planes", 1))
            aplanes = 1 if binary else abits
            ops = M * N * K * wplanes * aplanes * 2 / 32
            tops = ops / (gemv_ms * 1e-3) / 1e12
            roof = {"bound": "alu", "achieved": round(tops, 2), "peak": round(VALU_PEAK_TOPS, 2),
                    "unit": "Tlane-op/s", "frac": round(tops / VALU_PEAK_TOPS, 4)}
        roof["hbm_gbs"] = round(achieved, 2)
        roof["hbm_frac"] = round(achieved / HBM_PEAK_GBS, 4)
    traffic = None
    mt = MEASURED_TRAFFIC.get(args.workload + ("+fuse" if fuse else "")) if M == 1 else None
    if mt is not None and mt["kernels_sha256_16"] == kernels_sha():
        traffic = round(mt["bytes_per_launch"] / (gemv_ms * 1e-3) / 1e9, 2)

    out = {
        "metric": "packed-weight GB/s & % HBM peak, bit-plane GEMV 11008x4096 M=1; us/layer",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_layer": round(ms_per_step * 1e3, 3),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if fmt == "rabit" or (fmt == "sign" and not binary) else "int32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload} {N}x{K} M={M} ({'RaBiT 2-path residual binary, bf16 x' if fmt == 'rabit' else fmt})",
                   "N": N, "K": K, "M": M, "format": fmt, "packed_bytes": alg_bytes,
                   "seeds": {"W": synth.seed_for(synth.CONFIGS[data]["cfg"], si, synth.ROLE_W),
                             "x": synth.seed_for(synth.CONFIGS[data]["cfg"], si, synth.ROLE_X)},
                   "rotating_copies": copies, "rotating_bytes": copies * stride,
                   "graph_replay": graph is not None, "host_wall_s": round(wall, 4),
                   **({"weight_bits": wl["planes"], "act_bits": abits} if fmt == "wnam" else {}),
                   **({"fused_quantizer": True} if fuse else {}),
                   **({"rank": wl["rank"], "gemv_kernel_bytes": gemv_bytes} if hgf else {})},
        "roofline": {**roof, "traffic": traffic,
                     "traffic_bytes_per_launch": mt["bytes_per_launch"] if traffic is not None else None,
                     "kernel": ("gemv_xnor_kernel" if binary else
                                "gemv_sign_kernel" if fmt in ("rabit", "sign") else
                                "gemm_mfma_kernel" if mfma else "gemv_bits_nr_kernel"),
                     "kernel_us": round(gemv_ms * 1e3, 3)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and M == 1:
        try:
            out["cpu_baseline"] = cpu_baseline(wl)
        except Exception as e:  # reported, never fatal for the GPU figure
            out["cpu_baseline"] = {"error": repr(e)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
