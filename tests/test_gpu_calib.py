"""The DMPQ predictor calibration of Fig. 3 (6Bit-Diffusion), run through
the library: a one-linear residual block over drifting timesteps, Gamma_t
from block_gamma, E_rel_t of the NVFP4 and the INT8 activation path from
rel_err (quantized output against the bf16 output of the unquantized
linear), and (alpha, beta) per path from dmpq_fit.  The oracle repeats the
whole run on its own quantized outputs; Gamma agrees to summation order,
E_rel within the GEMM's float32 accumulation (1 %), the fit within 5 %."""
import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q
from oracle import tdc as T
from tests._gpu import dev, host, torch

pytestmark = pytest.mark.gpu

M = N = K = 256
STEPS = 6


def _trajectory():
    x = synth.activations(41, M, K, "normal", 4, 20.0)
    w = synth.weight(41, 0, N, K)
    xs = [x]
    for t in range(1, STEPS):
        # growing drift, so that Gamma spreads over the run
        xs.append(synth.drift(41, t, xs[-1], scale=0.05 * t))
    return xs, w


def test_calibration_run():
    qa, t = __import__("mixed_precision_quantized_act_amd"), torch()
    xs, w = _trajectory()
    wq = Q.nvfp4_encode(w)
    wd = Q.nvfp4_decode(*wq)
    ws_r = qa.workspace(qa.reduce_workspace(M * N))
    ws4 = qa.workspace(qa.qlinear_workspace(qa.NVFP4, M, N, K))
    ws8 = qa.workspace(qa.qlinear_workspace(qa.INT8, M, N, K))
    qws = qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, K))
    wq_d = [dev(wq[0]), dev(wq[1]), dev(np.array([wq[2]], np.float32))]
    g_gpu = np.zeros((STEPS, 1))
    e_gpu = np.zeros((STEPS, 2))
    g_or = np.zeros((STEPS, 1))
    e_or = np.zeros((STEPS, 2))
    for s, x in enumerate(xs):
        y_ref = F.f64_to_bf16_rne(G.linear_ref(F.bf16_to_f64(x), F.bf16_to_f64(w)))
        out = T.tdc_apply(x, y_ref)                         # block output in + Y
        xd, yrd = dev(x), dev(y_ref)
        sums = t.zeros(2, dtype=t.float64, device="cuda")
        qa.block_gamma(xd, dev(out), sums, ws_r)
        t.cuda.synchronize()
        g_gpu[s, 0] = qa.gamma_from_sums(host(sums))
        g_or[s, 0] = T.gamma(x, out)
        # NVFP4 activations
        aq, asc, ats = qa.empty_nvfp4(M, K, "cuda")
        qa.act_quant(qa.NVFP4, xd, aq, asc, ats, 0, qws)
        y4 = t.empty((M, N), dtype=t.bfloat16, device="cuda")
        qa.qlinear_nvfp4(aq, asc, ats, *wq_d, y4, M, N, K, ws=ws4)
        # INT8 activations
        a8, s8 = qa.empty_int8_act(M, K, "cuda")
        qa.act_quant(qa.INT8, xd, a8, s8)
        y8 = t.empty((M, N), dtype=t.bfloat16, device="cuda")
        qa.qlinear_int8(a8, s8, *wq_d[:2], wq_d[2], y8, M, N, K, ws=ws8)
        for j, y in enumerate((y4, y8)):
            qa.rel_err(y.view(t.int16), yrd, sums, ws_r)
            t.cuda.synchronize()
            e_gpu[s, j] = qa.rel_err_from_sums(host(sums))
        # the oracle's own quantized outputs
        a4o = Q.nvfp4_decode(*Q.nvfp4_encode(x))
        a8o = Q.int8_decode(*Q.int8_encode(x))
        for j, ad in enumerate((a4o, a8o)):
            yq = F.f64_to_bf16_rne(G.linear_ref(ad, wd))
            e_or[s, j] = T.rel_err(*T.rel_err_sums(yq, y_ref))
    assert np.allclose(g_gpu, g_or, rtol=1e-12, atol=0)
    assert np.allclose(e_gpu, e_or, rtol=1e-2, atol=0)
    assert np.all(e_gpu[:, 1] < e_gpu[:, 0])               # INT8 beats NVFP4 here
    a, b = qa.dmpq_fit(g_gpu, e_gpu, 2)
    ao, bo = T.calibrate(g_or, e_or, 2)
    pred, pred_o = a * g_gpu[:-1] + b, ao * g_or[:-1] + bo   # fitted E_rel over the run
    assert np.allclose(pred, pred_o, rtol=5e-2, atol=0)
