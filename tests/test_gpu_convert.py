"""Every finite float32 input of the element conversions the quantizers and
epilogues are built on (the library's test-only qa_test_convert), against
the oracle's rounding rules:

* E2M1 code of x as the NVFP4 encoders convert x * inv (6Bit-Diffusion,
  abstract: FP4 E2M1 elements) -- all finite float32, both signs;
* E4M3FN code of a group scale -- all non-negative finite float32;
* bf16 rounding of the epilogues -- all finite float32, both signs.

Method.  For x >= 0 the float32 bit pattern orders as the value, and each
rule (nearest representable value, ties to the even code, saturating) is a
non-decreasing step function of the pattern.  The library's outputs for
every non-negative finite pattern are read in chunks, and the patterns
where the output changes, with the outputs on both sides, must be exactly
the oracle's: its steps are located by bisection of the oracle's own
function (one search per output value).  Outputs of negative patterns must
be those of the positive pattern with the sign set.  In every chunk a
random sample is also compared with the oracle element by element.
"""
import numpy as np
import pytest

from oracle import formats as F
from tests._gpu import host, torch

pytestmark = pytest.mark.gpu

LAST_FINITE = 0x7F7FFFFF            # largest finite positive float32 pattern
CHUNK = 1 << 27


def _qa():
    import mixed_precision_quantized_act_amd as qa
    return qa


def _oracle(op, patterns):
    x = np.asarray(patterns, dtype=np.uint32).view(np.float32)
    if op == 0:
        return F.e2m1_encode(x).astype(np.int64)
    if op == 1:
        return F.e4m3_encode_nonneg(x).astype(np.int64)
    return F.f32_to_bf16_rne(x).astype(np.int64)


def _oracle_steps(op):
    """Patterns p in (0, LAST_FINITE] where the oracle's output differs from
    its output at p - 1, found by bisecting, for every output value v above
    the output at 0, for the first pattern whose output is >= v."""
    top = int(_oracle(op, [LAST_FINITE])[0])
    v = np.arange(int(_oracle(op, [0])[0]) + 1, top + 1, dtype=np.int64)
    lo = np.zeros(len(v), np.int64)                  # output(lo) < v
    hi = np.full(len(v), LAST_FINITE, np.int64)      # output(hi) >= v
    while np.any(hi - lo > 1):
        mid = (lo + hi) // 2
        ge = _oracle(op, mid) >= v
        hi = np.where(ge, mid, hi)
        lo = np.where(ge, lo, mid)
    return np.unique(hi)


def _device_outputs(op, first, count, buf):
    qa = _qa()
    qa._lib.convert_check(op, first, buf, count=count)
    torch().cuda.synchronize()
    out = host(buf[:count])                         # uint8, or int16 bits for bf16
    return out if op != 2 else out.view(np.uint16)


@pytest.mark.parametrize("op", [0, 1, 2])
def test_conversion_on_every_finite_float32(op):
    t = torch()
    rng = np.random.default_rng(op)
    buf = t.empty(CHUNK, dtype=t.int16 if op == 2 else t.uint8, device="cuda")
    sign = {0: 8, 2: 0x8000}.get(op)
    steps, before, after = [], [], []
    prev_last = None
    for first in range(0, LAST_FINITE + 1, CHUNK):
        count = min(CHUNK, LAST_FINITE + 1 - first)
        pos = _device_outputs(op, first, count, buf)
        if prev_last is None:
            assert int(pos[0]) == _oracle(op, [0])[0]
        elif int(pos[0]) != prev_last:
            steps.append(first)
            before.append(prev_last)
            after.append(int(pos[0]))
        d = np.flatnonzero(pos[1:] != pos[:-1]) + 1
        steps.extend((d + first).tolist())
        before.extend(pos[d - 1].astype(np.int64).tolist())
        after.extend(pos[d].astype(np.int64).tolist())
        prev_last = int(pos[-1])
        # a random sample of the chunk, element by element
        idx = rng.integers(0, count, 4096)
        np.testing.assert_array_equal(pos[idx].astype(np.int64), _oracle(op, first + idx))
        if sign is not None:
            neg = _device_outputs(op, 0x80000000 + first, count, buf)
            bad = np.flatnonzero(neg != (pos | pos.dtype.type(sign)))
            assert bad.size == 0, (op, hex(0x80000000 + first + int(bad[0])))
        print(f"[convert] op {op} patterns {first:#010x}+{count:#x}: {len(steps)} steps so far",
              flush=True)
    steps = np.array(steps, np.int64)
    want = _oracle_steps(op)
    np.testing.assert_array_equal(steps, want)
    np.testing.assert_array_equal(np.array(before), _oracle(op, want - 1))
    np.testing.assert_array_equal(np.array(after), _oracle(op, want))
