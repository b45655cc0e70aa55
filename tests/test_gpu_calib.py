"""The DMPQ predictor calibration of Fig. 3 (6Bit-Diffusion), run through
the library: a one-linear residual block over drifting timesteps, Gamma_t
from block_gamma, E_rel_t of the NVFP4 and the INT8 activation path from
rel_err (quantized output against the bf16 output of the unquantized
linear), and (alpha, beta) per path from dmpq_fit.  Each stage is checked
on its own inputs: Gamma and E_rel (rel_err on the library's own quantized
outputs) against the oracle's sums to summation order, the fit of the
library's E_rel bit for bit against the oracle's exact fit, the quantized
activations bit for bit.  The oracle also repeats the whole run on its own
quantized outputs: the two E_rel then differ by no more than the L2
distance of the two quantized outputs over the norm of the reference (the
triangle inequality), which is all that float32 against exact GEMM
accumulation leaves."""
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
    e_own = np.zeros((STEPS, 2))       # the oracle's rel_err on the library's outputs
    e_gap = np.zeros((STEPS, 2))       # ||y_lib - y_oracle|| / ||y_ref||
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
            e_own[s, j] = T.rel_err(*T.rel_err_sums(host(y), y_ref))
        # the oracle's own quantized activations (the library's, bit for bit)
        # and outputs
        e4, e8 = Q.nvfp4_encode(x), Q.int8_encode(x)
        np.testing.assert_array_equal(host(aq), e4[0])
        np.testing.assert_array_equal(host(asc), e4[1])
        assert host(ats)[0] == np.float32(e4[2])
        np.testing.assert_array_equal(host(a8), e8[0])
        np.testing.assert_array_equal(host(s8), e8[1])
        a4o, a8o = Q.nvfp4_decode(*e4), Q.int8_decode(*e8)
        ref = F.bf16_to_f64(y_ref)
        for j, (ad, y) in enumerate(((a4o, y4), (a8o, y8))):
            yq = F.f64_to_bf16_rne(G.linear_ref(ad, wd))
            e_or[s, j] = T.rel_err(*T.rel_err_sums(yq, y_ref))
            yl = F.bf16_to_f64(host(y))
            e_gap[s, j] = np.sqrt(np.sum((yl - F.bf16_to_f64(yq)) ** 2) / np.sum(ref ** 2))
    assert np.allclose(g_gpu, g_or, rtol=1e-12, atol=0)
    assert np.allclose(e_gpu, e_own, rtol=1e-12, atol=0)
    # end to end: |E_lib - E_oracle| <= ||y_lib - y_oracle|| / ||y_ref||
    # (plus the sums' own rounding), and that distance is small
    assert np.all(np.abs(e_gpu - e_or) <= e_gap * (1 + 1e-9) + 1e-12 * e_or)
    assert np.all(e_gap < 0.01 * e_or)
    assert np.all(e_gpu[:, 1] < e_gpu[:, 0])               # INT8 beats NVFP4 here
    a, b = qa.dmpq_fit(g_gpu, e_gpu, 2)
    ao, bo = T.calibrate(g_gpu, e_gpu, 2)
    assert np.array_equal(a, ao) and np.array_equal(b, bo)
    # and against the oracle's whole run: the fitted values are H e for the
    # least-squares hat matrix H of the x values (H = 1/n + xc xc^T / Sxx),
    # so inputs moved by at most eps move them by at most eps times H's
    # largest absolute row sum; float32 alpha and beta add their rounding
    ao2, bo2 = T.calibrate(g_or, e_or, 2)
    pred, pred_o = a * g_gpu[:-1] + b, ao2 * g_or[:-1] + bo2
    eps = np.max(np.abs(e_gpu - e_or)[1:], axis=0)
    xc = g_gpu[:-1, 0] - g_gpu[:-1, 0].mean()
    hat = 1.0 / len(xc) + np.outer(xc, xc) / np.sum(xc ** 2)
    bound = np.max(np.sum(np.abs(hat), axis=1)) * eps + \
        2.0 ** -22 * (np.abs(a * g_gpu[:-1]) + np.abs(b) + np.abs(ao2 * g_or[:-1]) + np.abs(bo2))
    assert np.all(np.abs(pred - pred_o) <= bound * (1 + 1e-6))
