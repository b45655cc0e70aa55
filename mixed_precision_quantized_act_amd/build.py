"""Build libqact.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run as ``python -m mixed_precision_quantized_act_amd.build`` or through
``__graft_entry__.build()``.  Each source compiles to its own object in
parallel (the GEMM sources hold many kernel instantiations), then one link
writes the library next to this file.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqact.so")
ROOT = os.path.dirname(HERE)
OBJ_DIR = os.path.join(HERE, "_build")

SOURCES = ["act_quant.hip", "qgemm.hip", "qgemm_i8.hip", "tdc.hip", "noalloc.hip", "convert_check.hip", "stage_ab.hip", "abi.cpp"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # exact float32 steps in the encoders: no contraction into FMA
    "-ffp-contract=off",
    # no packed-float32 instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + err)


def build(verbose=True):
    os.makedirs(OBJ_DIR, exist_ok=True)
    cc = hipcc()
    jobs = []
    for src in SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        jobs.append(([cc] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj], obj))
    if verbose:
        for cmd, _ in jobs:
            print(" ".join(cmd), flush=True)
    workers = max(1, min(len(jobs), os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(_run, [cmd for cmd, _ in jobs]))
    tmp = LIB + ".tmp"
    link = [cc, "--offload-arch=gfx950", "-shared", "-fPIC"] + [o for _, o in jobs] + ["-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    _run(link)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
