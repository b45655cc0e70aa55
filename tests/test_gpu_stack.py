"""Whole synthetic DiT stacks over 10 drifting timesteps (configs 4 and 5
shapes, and a small one), every step through libqact: DMPQ masks from the
previous step's Gamma (tau set at the first step with Gamma so that half of
the linears are INT8), TDC skips, act_quant, both GEMM paths, tdc_update
and tdc_apply.  Teacher-forced parity at every step for the checked blocks
(see tests/_stack.py); decisions for all blocks."""
import os
import sys
import time

import numpy as np
import pytest

import synth
from tests._gpu import dev
from tests._stack import Stack

pytestmark = pytest.mark.gpu

CASES = {
    "small": dict(cfg=1, L=4, H=256, F=1024, M=2048, check=(0, 3)),
    "cogvideox2b": dict(cfg=4, L=30, H=1920, F=7680, M=17776, check=(0, 29)),
    "cogvideox5b": dict(cfg=5, L=42, H=3072, F=12288, M=17776, check=(41,)),
}


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name", list(CASES))
def test_stack_teacher_forced(name):
    c = CASES[name]
    t0 = time.time()
    st = Stack(c["L"], c["H"], c["F"], c["M"], seed=1000 + c["cfg"], check_blocks=c["check"])
    for l in c["check"]:
        st.check_weights(l)
    x = synth.activations(c["cfg"], c["M"], c["H"], "normal")
    for t in range(10):
        x = synth.drift(c["cfg"], t, x)
        st.step(t, dev(x))
        _log(f"[stack {name}] step {t} pattern {st.pattern[-1]} int8 {st.masks[-1].mean():.2f} "
             f"checked {st.checked} {time.time() - t0:.1f}s")
    assert st.checked >= 4 * len(c["check"])
    # half of the linears go to INT8 at the step where tau was set
    assert 0.3 <= st.masks[1].mean() <= 0.7
    assert all(m.all() for m in st.masks[:1])            # no Gamma yet: all INT8
