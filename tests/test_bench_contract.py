"""Host-side checks of bench.py: the algorithmic byte counts behind
roofline.achieved, and the argument checks that end a run before any GPU
work (one GPU only; --tokens and --fuse only where the library has the path)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_packed_bytes_of_the_workloads():
    # planes 2 N K / 8 + g 2*2N + h 2*2K (RaBiT, 2 paths)
    assert bench.packed_bytes("rabit", 11008, 4096, 2) == 2 * 11008 * 4096 // 8 + 4 * 11008 + 4 * 4096 == 11332608
    # planes 2 N K / 8 + (delta, zero) fp16 per 128-group
    assert bench.packed_bytes("w2a8", 11008, 4096, 2) == 2 * 11008 * 4096 // 8 + 4 * 11008 * 4096 // 128 == 12681216
    # the GEMV kernel of an HGF layer reads the planes, gamma and B (A is read by the activation step)
    wl = bench.WORKLOADS["hgf"]
    assert bench.kernel_bytes(wl) == 2 * 4096 * 4096 // 8 + 4 + 2 * 32 * 4096


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr


@pytest.mark.parametrize("args", [("--workload", "rabit", "--tokens", "4"),
                                  ("--workload", "w2a8", "--tokens", "65"),
                                  ("--workload", "rabit", "--fuse"),
                                  ("--workload", "hgf", "--fuse"),
                                  ("--workload", "w2a8", "--tokens", "4", "--fuse")])
def test_unsupported_combinations_are_refused(args):
    r = _run(*args)
    assert r.returncode == 2, r.stderr
