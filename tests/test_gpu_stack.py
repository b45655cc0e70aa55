"""Whole synthetic DiT stacks over 10 drifting timesteps (configs 4 and 5
shapes, and a small one), every step through libqact: DMPQ masks from the
previous step's Gamma (tau set at the first step with Gamma so that half of
the linears are INT8), TDC skips, act_quant, both GEMM paths, tdc_update
and tdc_apply.  Teacher-forced parity at every step for the checked blocks
(see tests/_stack.py); decisions for all blocks.

At the configs' delta = 0.05 no block of these synthetic trajectories
skips (their successive Deltas differ by d of 0.07-0.55: quantization noise
of the activations, not the trained model's stability).  The "_skips" runs
set delta, from step 3 on, to the midpoint of the two middle d values the
blocks reported at step 2, so that about half of the eligible blocks skip
and the skip path (tdc_apply output and its Gamma sums, the Delta ring left
in place, the compute-after-skip rule) runs at full shape."""
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
    "cogvideox2b_skips": dict(cfg=4, L=30, H=1920, F=7680, M=17776, check=(0, 14, 29),
                              median_delta=True),
    "cogvideox5b_skips": dict(cfg=5, L=42, H=3072, F=12288, M=17776, check=(20, 41),
                              median_delta=True),
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
        if c.get("median_delta") and t == 2:
            d = np.sort(st.d_prev[np.isfinite(st.d_prev)])
            st.delta = float(0.5 * (d[(len(d) - 1) // 2] + d[len(d) // 2]))
        _log(f"[stack {name}] step {t} pattern {st.pattern[-1]} int8 {st.masks[-1].mean():.2f} "
             f"checked {st.checked} delta {st.delta:.4f} {time.time() - t0:.1f}s")
    assert st.checked >= 4 * len(c["check"])
    if c.get("median_delta"):
        # skips happened, on checked blocks too, and every skip was followed
        # by a computed step (a block skipped at t-1 computes at t)
        pat = np.array([list(p) for p in st.pattern])
        assert (pat == "S").sum() >= len(pat[0]) // 2
        assert any((pat[:, l] == "S").any() for l in c["check"])
        for l in range(pat.shape[1]):
            col = "".join(pat[:, l])
            assert "SS" not in col and col[:2] == "CC"
    # half of the linears go to INT8 at the step where tau was set
    assert 0.3 <= st.masks[1].mean() <= 0.7
    assert all(m.all() for m in st.masks[:1])            # no Gamma yet: all INT8
