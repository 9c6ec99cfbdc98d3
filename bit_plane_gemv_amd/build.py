"""Build libbitq.so in-tree with hipcc for gfx950.

    python bit_plane_gemv_amd/build.py          # build (always recompiles)
    python bit_plane_gemv_amd/build.py --asm    # also dump the gfx950 assembly

This file is loaded by path (not as part of the package), so it works before
libbitq.so exists; importing the package itself requires the built library.

The shared library holds the host code (validation, packer, quantizers) and
the HIP kernels.  Host code is compiled without floating-point contraction so
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
]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=off",
          f"-I{os.path.join(HERE, '..', 'include')}"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("command failed: " + " ".join(cmd))
    return r


def build(asm: bool = False, verbose: bool = False) -> str:
    objs = []
    host_src = os.path.join(CSRC, "bitq_host.cpp")
    kern_src = os.path.join(CSRC, "bitq_kernels.hip")
    host_obj = os.path.join(CSRC, "bitq_host.o")
    kern_obj = os.path.join(CSRC, "bitq_kernels.o")
    _run([HIPCC, *COMMON, "-c", host_src, "-o", host_obj])
    objs.append(host_obj)
    _run([HIPCC, *COMMON, *DEVICE_FLAGS, "-x", "hip", "-c", kern_src, "-o", kern_obj])
    objs.append(kern_obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    if asm:
        out = os.path.join(CSRC, f"bitq_kernels-hip-amdgcn-amd-amdhsa-{ARCH}.s")
        _run([HIPCC, *COMMON, *DEVICE_FLAGS, "-x", "hip", "--cuda-device-only", "-S",
              kern_src, "-o", out])
        if verbose:
            print("assembly:", out)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(asm="--asm" in sys.argv, verbose=True)
