"""Build libbitq.so in-tree with hipcc for gfx950.

    python bit_plane_gemv_amd/build.py          # build (always recompiles)
    python bit_plane_gemv_amd/build.py --asm    # also dump the gfx950 assembly
    python bit_plane_gemv_amd/build.py --sanitize   # host code under ASan/UBSan

This file is loaded by path (not as part of the package), so it works before
libbitq.so exists; importing the package itself requires the built library.

The shared library holds the host code (validation, packer, quantizers) and
the HIP kernels (one source per kernel family, compiled in parallel).  Host code is compiled without floating-point contraction so
that the offline quantizers follow the documented arithmetic order.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbitq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

DEVICE_FLAGS = [
    f"--offload-arch={ARCH}",
    # code object v5: loadable by the HIP runtime torch ships as well as ROCm 7.2's
    "-mcode-object-version=5",
    # keep the compiler from emitting packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first 16 kernel-argument dwords arrive in scalar registers instead
    # of through scalar loads at the start of every kernel (measured 0.3 -
    # 0.4 us per launch on the decode GEMVs)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=off",
          f"-I{os.path.join(HERE, '..', 'include')}"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("command failed: " + " ".join(cmd))
    return r


def _run_all(cmds, jobs: int):
    """Run the compile commands, at most `jobs` at a time; raise on the first failure."""
    pending, running = list(cmds), []
    failed = None
    while pending or running:
        while pending and len(running) < jobs and failed is None:
            cmd = pending.pop(0)
            running.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                                  text=True)))
        cmd, p = running.pop(0)
        out, _ = p.communicate()
        if p.returncode != 0 and failed is None:
            sys.stderr.write(out)
            failed = cmd
        if failed is not None:
            pending.clear()
    if failed is not None:
        raise RuntimeError("command failed: " + " ".join(failed))


def kernel_sources() -> list:
    """The HIP sources of the library (one per kernel family)."""
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(asm: bool = False, verbose: bool = False, jobs: int | None = None) -> str:
    jobs = jobs or max(1, min(8, os.cpu_count() or 1))
    host_src = os.path.join(CSRC, "bitq_host.cpp")
    cmds, objs = [], []
    host_obj = os.path.join(CSRC, "bitq_host.o")
    cmds.append([HIPCC, *COMMON, "-c", host_src, "-o", host_obj])
    objs.append(host_obj)
    for src in kernel_sources():
        obj = src[:-4] + ".o"
        cmds.append([HIPCC, *COMMON, *DEVICE_FLAGS, "-x", "hip", "-c", src, "-o", obj])
        objs.append(obj)
    # the largest sources first, so that they start early
    cmds.sort(key=lambda c: -os.path.getsize(c[-3]))
    _run_all(cmds, jobs)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    if asm:
        for src in kernel_sources():
            out = src[:-4] + f"-hip-amdgcn-amd-amdhsa-{ARCH}.s"
            _run([HIPCC, *COMMON, *DEVICE_FLAGS, "-x", "hip", "--cuda-device-only", "-S", src, "-o", out])
            if verbose:
                print("assembly:", out)
    if verbose:
        print("built", LIB)
    return LIB


SAN_LIB = os.path.join(HERE, "libbitq_san.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def build_sanitized(verbose: bool = False, jobs: int | None = None) -> str:
    """libbitq_san.so: the host code (validation, packer, quantizers) built by
    g++ with AddressSanitizer and UndefinedBehaviorSanitizer, linked with the
    ordinary gfx950 kernel objects.  For the CPU test suite:

        python bit_plane_gemv_amd/build.py --sanitize
        ASAN_OPTIONS=detect_leaks=0 LD_PRELOAD=$(g++ -print-file-name=libasan.so) \
            BITQ_LIBRARY=bit_plane_gemv_amd/libbitq_san.so python -m pytest tests -m "not gpu"

    The kernels themselves are not instrumented (device code); only host code is."""
    jobs = jobs or max(1, min(8, os.cpu_count() or 1))
    host_src = os.path.join(CSRC, "bitq_host.cpp")
    host_obj = os.path.join(CSRC, "bitq_host_san.o")
    inc = f"-I{os.path.join(HERE, '..', 'include')}"
    cmds = [["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off", "-D__HIP_PLATFORM_AMD__", inc,
             "-I/opt/rocm/include", *SAN_FLAGS, "-c", host_src, "-o", host_obj]]
    objs = [host_obj]
    for src in kernel_sources():
        obj = src[:-4] + "_san.o"
        cmds.append([HIPCC, *COMMON, *DEVICE_FLAGS, "-x", "hip", "-c", src, "-o", obj])
        objs.append(obj)
    _run_all(cmds, jobs)
    tmp = SAN_LIB + ".tmp"
    _run(["g++", "-shared", *SAN_FLAGS, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-o", tmp])
    os.replace(tmp, SAN_LIB)
    for o in objs:
        os.remove(o)
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        build_sanitized(verbose=True)
    else:
        build(asm="--asm" in sys.argv, verbose=True)
