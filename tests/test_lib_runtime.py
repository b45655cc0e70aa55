"""The binding leaves one HIP runtime in the process.  torch ships its own
libamdhip64 (and HSA runtime) and its libraries ask for it by the name
libamdhip64.so; libqact.so asks for libamdhip64.so.7.  Loaded before
torch, the library would pull in a second runtime beside torch's, and the
one that reaches the GPU second finds no device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROBE = r"""
import sys
sys.path.insert(0, {root!r})
import mixed_precision_quantized_act_amd as qa
qa.lib()                      # the library first, torch only afterwards
import torch  # noqa: F401
paths = set()
for line in open("/proc/self/maps"):
    parts = line.split()
    if len(parts) >= 6 and ("libamdhip64" in parts[5] or "libhsa-runtime64" in parts[5]):
        paths.add(parts[5])
print(len([p for p in paths if "libamdhip64" in p]), len([p for p in paths if "hsa-runtime" in p]))
"""


def test_one_hip_runtime_when_library_loads_first():
    r = subprocess.run([sys.executable, "-c", PROBE.format(root=ROOT)], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    hip, hsa = map(int, r.stdout.split()[-2:])
    assert (hip, hsa) == (1, 1), r.stdout
