"""The GEMM kernels' tile order and K split (csrc/tile_order.h, the same
source the kernels compile) built for the host and run over every
workgroup of every launch mode for ~100k shapes: each output tile, and each
K unit of a split tile, is reached exactly once and in bounds."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixed_precision_quantized_act_amd", "csrc")


def test_tile_order_host_build(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "tile_order_check"
    subprocess.run([cxx, "-O2", "-std=c++17", "-Wall", "-Werror", "-I", CSRC,
                    os.path.join(ROOT, "tests", "tile_order_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:]
    assert "0 failures" in r.stdout
