#!/usr/bin/env python3
"""Benchmark of the bit-plane GEMV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one batch-1 GEMV y = W^ x over one Llama-2-7B gate/up layer
(11008 x 4096): the RaBiT 2-path residual-binary layer by default (the
workload the headline metric is quoted on).  The default run also measures
the same layer in the W2A8 bit-plane format (the activation quantizer plus
the AND+popcount GEMV, and the GEMV with the quantizer fused into it) and
reports it under the key "w2a8".  --workload picks another layer (the table
WORKLOADS); --tokens M (integer formats, 2..64) runs the small-M path
instead: M tokens per step, each weight read once, and the roofline is then
the contraction's (int8 matrix cores from the library's switch on, else VALU
lane-operations).

Measurement:
  * The packed layer is replicated into >= 1 GiB of distinct device copies and
    step i reads copy i mod C, so every step streams its weights from HBM
    (the 256 MB Infinity Cache and the L2s cannot hold the rotation).
  * Inputs are resident in HBM before timing starts.  The K timed steps are
    captured once into a HIP graph (up to 64 steps: launched one by one).  A
    bounded wait kernel is queued ahead of them, so the GPU starts the first
    step only once the host has submitted them all; HIP events recorded on
    the launch stream bracket the steps.  The measured time is GPU time of
    the K steps.
  * value = packed weight bytes x K / elapsed (GB/s).  roofline.achieved is
    the algorithmic bytes of the product kernel divided by its per-launch time,
    measured the same way on a graph of that kernel alone.
  * roofline.floor_us and empty_us come from two context kernels of the
    library, timed the same way on the same rotation: one that only streams
    the same bytes with the product kernel's grid (and writes one fp32 per
    output row), and one that does nothing with that grid.  frac_of_floor =
    floor_us / kernel_us.
  * cpu_baseline: the CPU oracle (explicit fp64 dequantization + dot product)
    on the same layer, timed on the host for a bounded number of repetitions.
"""
from __future__ import annotations

import argparse
import hashlib
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
MFMA_MIN_TOKENS = {"w2a8": 2, "wnam": 2, "ternary": 3}  # the library's switch to the matrix cores
ROTATE_BYTES = 1 << 30
CSRC = os.path.join(ROOT, "bit_plane_gemv_amd", "csrc")
METRIC = "packed-weight GB/s & % HBM peak, bit-plane GEMV 11008x4096 M=1; us/layer"

# HBM bytes moved per launch of a product kernel, from rocprofv3 counter runs
# (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0; factors calibrated on a plain copy
# kernel of known size; profiles/ holds the runs).  Each entry is valid only
# for the kernel source and the build script it was measured with (first 16
# hex digits of the sha256 of each file); otherwise traffic is reported as null.
MEASURED_TRAFFIC: dict = {
    "rabit": {"source": "bitq_sign.hip", "sha16": "ba906aeaa6be2c6a", "build_sha16": "75709457503c2a5c",
              "bytes_per_launch": 13458432, "profile": "profiles/gemv_sign_kernel_rabit_11008x4096.md"},
    "w2a8": {"source": "bitq_bits.hip", "sha16": "241574416dea4db5", "build_sha16": "75709457503c2a5c",
             "bytes_per_launch": 12822528, "profile": "profiles/gemv_bits_nr_kernel_w2a8_11008x4096.md"},
    "w2a8+fuse": {"source": "bitq_bits.hip", "sha16": "241574416dea4db5", "build_sha16": "75709457503c2a5c",
                  "bytes_per_launch": 12880896, "profile": "profiles/gemv_bits_nr_kernel_fused_w2a8_11008x4096.md"},
}
BUILD_SCRIPT = os.path.join(ROOT, "bit_plane_gemv_amd", "build.py")


def source_sha(name: str) -> str:
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def build_sha() -> str:
    with open(BUILD_SCRIPT, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(key: str):
    mt = MEASURED_TRAFFIC.get(key)
    if mt is None or mt["sha16"] != source_sha(mt["source"]) or mt["build_sha16"] != build_sha():
        return None
    return mt


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


def host_description() -> dict:
    """The host the CPU baseline ran on: CPU model, logical CPUs, CPUs in
    this process's affinity mask, and the BLAS thread pools."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    blas = []
    try:
        from threadpoolctl import threadpool_info
        blas = [{"api": i.get("user_api"), "lib": i.get("internal_api"), "threads": i.get("num_threads")}
                for i in threadpool_info()]
    except Exception:
        pass
    return {"cpu_model": model, "cpu_count": os.cpu_count(), "affinity_cpus": affinity, "blas": blas,
            "env_threads": {k: os.environ[k] for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
                            if k in os.environ}}


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
    blas_gemm = True   # the fp64 dot is a BLAS matmul (threads = the BLAS pool)
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
    host = host_description()
    threads = max([b["threads"] or 1 for b in host["blas"]] or [1])
    if host["affinity_cpus"]:
        threads = min(threads, host["affinity_cpus"])
    times = []
    t_all = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        run()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all > budget_s or len(times) >= 50:
            break
    med = float(np.median(times))
    return {"value": round(packed_bytes(fmt, N, K, wl.get("planes", 2), wl.get("rank", 0)) / med / 1e9, 4),
            "unit": "GB/s",
            "cores": int(threads) if blas_gemm else 1,
            "kind": "oracle",
            "sample": f"{what}, {fmt} {N}x{K} M=1, one GEMV per run, {len(times)} runs in "
                      f"{time.perf_counter() - t_all:.1f} s, median {med * 1e3:.1f} ms per GEMV",
            "us_per_gemv": round(med * 1e6, 1),
            "host": host}


class Timer:
    """Per-step GPU time of a sequence of K steps captured in one HIP graph.

    The graph is replayed once untimed.  For the timed replay a bounded wait
    kernel (bitq_ctx_spin) is queued first, long enough to cover the host's
    submission of the graph, so the first step starts right after the start
    event and the events measure GPU time only.

    Up to DIRECT_MAX_STEPS steps are launched one by one instead, behind the
    same wait kernel (sized from an untimed run of the same launches): a
    graph replay adds about 4 us of its own start-up to the events' fixed
    cost of about 8 us, which a short region would divide among few steps
    (RaBiT 11008x4096, 20 steps: 6.09 us per step launched directly, 6.33 us
    from a graph, 5.68 us at 2000 steps)."""

    DIRECT_MAX_STEPS = 64

    def __init__(self, torch, bq, graph: bool = True):
        self.torch, self.bq, self.graph = torch, bq, graph

    def _direct_ms(self, step, K: int, warmup: int) -> float:
        # Step indices select the weight copy (i mod the rotation): the
        # untimed run reads copies W + K .. W + 2K - 1, the timed run
        # W .. W + K - 1, so the timed steps do not re-read weights that the
        # untimed run or the warmup (0 .. W - 1) have just brought into the
        # caches.
        torch, bq = self.torch, self.bq
        stream = torch.cuda.current_stream()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):                  # untimed; measures the host's launch time
            step(warmup + K + i, stream)
        host_us = (time.perf_counter() - t0) * 1e6
        torch.cuda.synchronize()
        spin_us = int(min(10000, max(300, 3 * host_us + 100)))
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        bq.ctx_spin(spin_us, stream=stream)
        ev0.record(stream)
        t0 = time.perf_counter()
        for i in range(K):
            step(warmup + i, stream)
        ev1.record(stream)
        host2_us = (time.perf_counter() - t0) * 1e6
        torch.cuda.synchronize()
        if host2_us > spin_us:              # the wait did not cover the launches: use a graph
            return None
        return ev0.elapsed_time(ev1) / K

    def per_step_ms(self, step, K: int, warmup: int) -> float:
        torch, bq = self.torch, self.bq
        for i in range(warmup):
            step(i, torch.cuda.current_stream())
        torch.cuda.synchronize()
        if not self.graph:        # launched one by one from the host (for counter runs)
            stream = torch.cuda.current_stream()
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for i in range(K):
                step(i, stream)
            ev1.record(stream)
            torch.cuda.synchronize()
            return ev0.elapsed_time(ev1) / K
        if K <= self.DIRECT_MAX_STEPS:
            ms = self._direct_ms(step, K, warmup)
            if ms is not None:
                return ms
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                st = torch.cuda.current_stream()
                for i in range(K):
                    step(i, st)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()                          # untimed; also measures the host submission time
        host_us = (time.perf_counter() - t0) * 1e6
        torch.cuda.synchronize()
        spin_us = int(min(10000, max(200, 2 * host_us + 100)))
        stream = torch.cuda.current_stream()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        bq.ctx_spin(spin_us, stream=stream)
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        del g
        return ev0.elapsed_time(ev1) / K


class Layer:
    """One workload layer on the device: the rotation of packed copies, the
    activations and the buffers of its steps."""

    def __init__(self, torch, bq, synth, wl: dict, M: int):
        self.wl, self.M = wl, M
        self.fmt, self.N, self.K, si = wl["fmt"], wl["N"], wl["K"], wl["shape_idx"]
        N, K = self.N, self.K
        dev = torch.device("cuda:0")
        self.bq = bq
        t0 = time.perf_counter()
        data = wl.get("data", self.fmt)
        self.data = data
        W = synth.weights(data, si, N, K)
        self.desc = bq.wdesc(self.fmt, N, K, planes=wl.get("planes"), abits=wl.get("abits"), rank=wl.get("rank"))
        self.abits = wl.get("abits", 8)
        self.hgf = self.fmt == "hgf"
        if self.hgf:
            Ab, Bb, alpha = synth.lora_params(si, N, K, wl["rank"])
            blob = bq.quantize_weights_hgf(self.desc, W, Ab, Bb, alpha)
        else:
            blob = bq.quantize_weights(self.desc, W, bit_balance=bool(wl.get("bit_balance")))
        log(f"quantized+packed {self.fmt} {N}x{K} in {time.perf_counter() - t0:.1f}s, blob {blob.nbytes} B")
        self.alg_bytes = packed_bytes(self.fmt, N, K, wl.get("planes", 2), wl.get("rank", 0))
        self.gemv_bytes = kernel_bytes(wl)
        self.copies = max(2, math.ceil(ROTATE_BYTES / blob.nbytes))
        base = torch.empty(blob.nbytes, dtype=torch.uint8, device=dev)
        base.copy_(torch.from_numpy(blob))
        self.stride = (blob.nbytes + 4095) // 4096 * 4096
        self.pool = torch.empty(self.copies * self.stride, dtype=torch.uint8, device=dev)
        for c in range(self.copies):
            self.pool[c * self.stride:c * self.stride + blob.nbytes].copy_(base)
        del base
        self.blobs = [self.pool[c * self.stride:c * self.stride + blob.nbytes] for c in range(self.copies)]
        xs, _ = synth.activations(data, si, M, K)
        if xs.dtype == np.float32:      # fp32 activations (the sign workloads' inputs)
            self.x, self.x_dt = torch.from_numpy(np.ascontiguousarray(xs)).to(dev), bq.DT_F32
        else:                           # bf16 bit patterns
            self.x, self.x_dt = torch.from_numpy(np.ascontiguousarray(xs).view(np.int16)).to(dev), bq.DT_BF16
        self.y = torch.empty(M * N, dtype=torch.float32, device=dev)
        self.ws = torch.zeros(bq.workspace_size(self.desc, M), dtype=torch.uint8, device=dev)
        self.binary = bool(wl.get("binary"))
        self.integer = self.fmt in ("ternary", "w2a8", "bvsr", "wnam", "hgf") or self.binary
        if self.binary:
            self.act = torch.zeros(bq.binact_size(M, K), dtype=torch.uint8, device=dev)
        elif self.hgf:
            act_bytes, act_ws_bytes = bq.hgf_act_size(self.desc, M)
            self.act = torch.zeros(act_bytes, dtype=torch.uint8, device=dev)
            self.act_ws = torch.zeros(act_ws_bytes, dtype=torch.uint8, device=dev)
        else:
            self.act = torch.zeros(bq.act_size(M, K), dtype=torch.uint8, device=dev) if self.integer else None
        self.act_dt = bq.DT_BINARY if self.binary else bq.DT_ACT
        self.seeds = {"W": synth.seed_for(synth.CONFIGS[data]["cfg"], si, synth.ROLE_W),
                      "x": synth.seed_for(synth.CONFIGS[data]["cfg"], si, synth.ROLE_X)}

    # ---- the pieces of a step
    def activation_step(self, st):
        bq = self.bq
        if self.binary:
            bq.binarize_act(self.x, self.x_dt, self.M, self.K, self.act, stream=st)
        elif self.hgf:
            bq.quantize_act_hgf(self.desc, self.blobs[0], self.x, self.x_dt, self.M, self.act, self.act_ws, stream=st)
        else:
            bq.quantize_act(self.x, self.x_dt, self.M, self.K, self.act, stream=st, abits=self.abits)

    def product(self, i, st):
        """The GEMV (one token) or the small-M GEMM (M tokens) on copy i."""
        bq, w = self.bq, self.blobs[i % self.copies]
        if not self.integer:
            bq.gemv(self.desc, w, self.x, self.x_dt, self.y, self.ws, stream=st)
        elif self.M == 1:
            bq.gemv(self.desc, w, self.act, self.act_dt, self.y, None if self.binary else self.ws, stream=st)
        else:
            bq.gemm_smallM(self.desc, w, self.act, self.M, self.y, None if self.binary else self.ws, stream=st)

    def step(self, i, st):
        if self.integer:
            if self.hgf:   # the activation step reads A from the copy this step uses
                self.bq.quantize_act_hgf(self.desc, self.blobs[i % self.copies], self.x, self.x_dt, self.M,
                                         self.act, self.act_ws, stream=st)
            else:
                self.activation_step(st)
        self.product(i, st)

    def fused_step(self, i, st):
        self.bq.gemv(self.desc, self.blobs[i % self.copies], self.x, self.x_dt, self.y, None,
                     flags=self.bq.F_FUSE_QUANT, stream=st)

    def context_floor(self, timer: Timer, K: int, warmup: int, nbytes: int, fused: bool = False) -> dict:
        """Per-launch time of the stream-read and empty context kernels with
        the product kernel's grid, over the same rotation."""
        bq = self.bq
        flags = bq.F_FUSE_QUANT if fused else 0
        x_dt = self.x_dt if (fused or not self.integer) else self.act_dt
        grid, block = bq.ctx_launch_shape(self.desc, self.M, x_dt, flags)
        n16 = nbytes // 16 * 16
        floor_ms = timer.per_step_ms(
            lambda i, st: bq.ctx_stream(self.blobs[i % self.copies], n16, grid, self.y, self.N, stream=st),
            K, warmup)
        empty_ms = timer.per_step_ms(lambda i, st: bq.ctx_empty(grid, stream=st), K, warmup)
        return {"floor_us": round(floor_ms * 1e3, 3), "empty_us": round(empty_ms * 1e3, 3),
                "floor_bytes": n16, "grid": grid, "block": block}


def hbm_roofline(nbytes: int, us: float, kernel: str, ctx: dict | None, traffic_key: str | None) -> dict:
    achieved = nbytes / (us * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "traffic_bytes_per_launch": None,
            "kernel": kernel, "kernel_us": round(us, 3), "alg_bytes": nbytes}
    mt = measured_traffic(traffic_key) if traffic_key else None
    if mt is not None:
        roof["traffic"] = round(mt["bytes_per_launch"] / (us * 1e-6) / 1e9, 2)
        roof["traffic_bytes_per_launch"] = mt["bytes_per_launch"]
    if ctx is not None:
        roof.update(ctx)
        roof["frac_of_floor"] = round(ctx["floor_us"] / us, 4)
    return roof


def product_kernel_name(layer: Layer, mfma: bool) -> str:
    if layer.binary:
        return "gemv_xnor_kernel"
    if layer.fmt in ("rabit", "sign"):
        return "gemv_sign_kernel"
    return "gemm_mfma_kernel" if mfma else "gemv_bits_nr_kernel"


def w2a8_headline(torch, bq, synth, timer: Timer, K_steps: int, warmup: int, cpu: bool) -> dict:
    """The W2A8 11008x4096 M=1 layer: GEMV kernel alone, the two-launch step
    (quantizer + GEMV) and the fused step, each with its roofline."""
    wl = WORKLOADS["w2a8"]
    L = Layer(torch, bq, synth, wl, 1)
    gemv_ms = timer.per_step_ms(L.product, K_steps, warmup)
    step_ms = timer.per_step_ms(L.step, K_steps, warmup)
    fused_ms = timer.per_step_ms(L.fused_step, K_steps, warmup)
    ctx = L.context_floor(timer, K_steps, warmup, L.gemv_bytes)
    ctx_f = L.context_floor(timer, K_steps, warmup, L.gemv_bytes, fused=True)
    out = {
        "workload": f"w2a8 {L.N}x{L.K} M=1 (2-bit asymmetric weights, group 128, int8 per-token activations)",
        "packed_bytes": L.alg_bytes,
        "gemv": {"us": round(gemv_ms * 1e3, 3), "GB/s": round(L.alg_bytes / (gemv_ms * 1e-3) / 1e9, 2),
                 "roofline": hbm_roofline(L.gemv_bytes, gemv_ms * 1e3, "gemv_bits_nr_kernel", ctx, "w2a8")},
        "step_two_launch": {"us": round(step_ms * 1e3, 3),
                            "GB/s": round(L.alg_bytes / (step_ms * 1e-3) / 1e9, 2),
                            "kernels": ["quant_act_kernel", "gemv_bits_nr_kernel"]},
        "fused_step": {"us": round(fused_ms * 1e3, 3), "GB/s": round(L.alg_bytes / (fused_ms * 1e-3) / 1e9, 2),
                       "roofline": hbm_roofline(L.gemv_bytes, fused_ms * 1e3, "gemv_bits_nr_kernel (fused quantizer)",
                                                ctx_f, "w2a8+fuse")},
        "seeds": L.seeds, "rotating_copies": L.copies,
    }
    del L
    torch.cuda.empty_cache()
    if cpu:
        try:
            out["cpu_baseline"] = cpu_baseline(wl, budget_s=8.0)
        except Exception as e:  # reported, never fatal for the GPU figure
            out["cpu_baseline"] = {"error": repr(e)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="rabit", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-second", action="store_true", help="skip the W2A8 headline of the default run")
    ap.add_argument("--no-context", action="store_true", help="skip the context kernels (floor, empty)")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every step from the host instead of a graph replay (for profiler counter runs; "
                         "the per-step time then includes host launch gaps)")
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
    wl = WORKLOADS[args.workload]
    fmt = wl["fmt"]
    M = args.tokens
    if M != 1 and (fmt in ("rabit",) or (fmt == "sign" and not wl.get("binary")) or not 1 <= M <= 64):
        print("--tokens > 1 needs an integer-activation workload and at most 64 tokens", file=sys.stderr)
        sys.exit(2)
    fuse = args.fuse
    if fuse and (M != 1 or fmt not in ("ternary", "w2a8", "bvsr", "wnam") or wl.get("binary")):
        print("--fuse needs one token and a TERNARY/W2A8/BVSR4/WNAM workload", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_plane_gemv_amd as bq
    import synth

    torch.cuda.set_device(torch.device("cuda:0"))
    timer = Timer(torch, bq, graph=not args.no_graph)
    L = Layer(torch, bq, synth, wl, M)
    K_steps = args.steps
    N, K = L.N, L.K

    # ---- the timed steps (the contract's K steps)
    step = L.fused_step if fuse else L.step
    t_wall = time.perf_counter()
    ms_per_step = timer.per_step_ms(step, K_steps, args.warmup)
    wall = time.perf_counter() - t_wall
    value = L.alg_bytes / (ms_per_step * 1e-3) / 1e9

    # ---- the product kernel alone (integer workloads also run an activation
    #      step in each two-launch step)
    kernel_ms = ms_per_step
    if L.integer and not fuse:
        kernel_ms = timer.per_step_ms(L.product, K_steps, args.warmup)
    mfma = fmt in MFMA_MIN_TOKENS and M >= MFMA_MIN_TOKENS[fmt]
    kname = product_kernel_name(L, mfma) + (" (fused quantizer)" if fuse else "")
    ctx = None if args.no_context else L.context_floor(timer, K_steps, args.warmup, L.gemv_bytes, fused=fuse)
    traffic_key = (args.workload + ("+fuse" if fuse else "")) if M == 1 else None
    roof = hbm_roofline(L.gemv_bytes, kernel_ms * 1e3, kname, ctx, traffic_key)
    if M > 1:
        # the small-M contraction: int8 ops (2 M N K) on the matrix cores, or,
        # on the VALU, the AND and popcount lane-operations of the bit planes
        # (2 per weight plane x activation plane x 32 weights x token)
        hbm = roof
        if mfma:
            tops = 2.0 * M * N * K / (kernel_ms * 1e-3) / 1e12
            roof = {"bound": "mfma", "achieved": round(tops, 2), "peak": INT8_MFMA_PEAK_TOPS, "unit": "TOP/s",
                    "frac": round(tops / INT8_MFMA_PEAK_TOPS, 4)}
        else:
            wplanes = {"ternary": 2, "w2a8": 2, "bvsr": 4, "hgf": 2}.get(fmt, wl.get("planes", 1))
            aplanes = 1 if L.binary else L.abits
            ops = M * N * K * wplanes * aplanes * 2 / 32
            tops = ops / (kernel_ms * 1e-3) / 1e12
            roof = {"bound": "alu", "achieved": round(tops, 2), "peak": round(VALU_PEAK_TOPS, 2),
                    "unit": "Tlane-op/s", "frac": round(tops / VALU_PEAK_TOPS, 4)}
        roof.update({"kernel": kname, "kernel_us": hbm["kernel_us"], "hbm_gbs": hbm["achieved"],
                     "hbm_frac": hbm["frac"], "traffic": None})
        for k in ("floor_us", "empty_us", "frac_of_floor", "grid", "block"):
            if k in hbm:
                roof[k] = hbm[k]

    out = {
        "metric": METRIC,
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
        "dtype": "f32" if fmt == "rabit" or (fmt == "sign" and not L.binary) else "int32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload} {N}x{K} M={M} "
                               f"({'RaBiT 2-path residual binary, bf16 x' if fmt == 'rabit' else fmt})",
                   "N": N, "K": K, "M": M, "format": fmt, "packed_bytes": L.alg_bytes, "seeds": L.seeds,
                   "rotating_copies": L.copies, "rotating_bytes": L.copies * L.stride,
                   "graph_replay": not args.no_graph, "host_wall_s": round(wall, 4),
                   **({"weight_bits": wl["planes"], "act_bits": L.abits} if fmt == "wnam" else {}),
                   **({"fused_quantizer": True} if fuse else {}),
                   **({"rank": wl["rank"], "gemv_kernel_bytes": L.gemv_bytes} if L.hgf else {})},
        "roofline": roof,
        "cpu_baseline": None,
    }
    del L
    torch.cuda.empty_cache()
    if args.workload == "rabit" and M == 1 and not fuse and not args.no_second:
        out["w2a8"] = w2a8_headline(torch, bq, synth, timer, K_steps, args.warmup, not args.no_cpu_baseline)
    if not args.no_cpu_baseline and M == 1:
        try:
            out["cpu_baseline"] = cpu_baseline(wl)
        except Exception as e:  # reported, never fatal for the GPU figure
            out["cpu_baseline"] = {"error": repr(e)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
