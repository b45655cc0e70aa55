"""The FFN configuration at its full size (17776 Student-t(3) tokens,
1920 -> 7680 GELU-tanh -> 1920, NVFP4 weights) with its DMPQ mask.

The pages fit the predictor p = alpha Gamma_{t-1} + beta per internal linear
(Fig. 3 caption) and keep INT8 for the volatile layers (abstract); the
configuration asks for alpha = 1, beta = 0.01 and a threshold that sends
about half of the linears to INT8.  One FFN has a single input/output pair,
so its two linears share one Gamma: the FFN is run as a residual block
(out = in + Down(GELU(Up(in)))) over 10 timesteps of the drift
x_t = x_{t-1} + 0.02 N(0,1), and tau is the midpoint of the two middle
predictions of a calibration pass (every linear INT8, as at t = 0) over all
(step, linear) pairs.  The DMPQ pass then takes each step's format from its
own Gamma_{t-1}.  Checked against the oracle, teacher-forced: the masks at
every step (bit-exact), and at steps 0, 1 and the first step of each format
after it the activation codes and scales of both linears (bit-exact, on
sampled rows, the hidden activation's tensor scale from the whole tensor),
both linears' outputs (rel. Frobenius <= 1e-3), the residual add
(bit-exact) and the Gamma sums (1e-12).
"""
import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q
from oracle import tdc as T
from tests._gpu import dev, host, rel_fro, sample_rows, torch

pytestmark = pytest.mark.gpu

STEPS = 10
ALPHA, BETA = 1.0, 0.01


def _qa():
    import mixed_precision_quantized_act_amd as qa
    return qa


class FFNBlock:
    def __init__(self):
        qa, t = _qa(), torch()
        x0, wu, wd = synth.ffn_case(3)
        self.x0 = x0
        self.M, self.K = x0.shape
        self.F = wu.shape[0]
        self.w = []
        for w in (wu, wd):
            N, K = w.shape
            q, s, ts = qa.empty_nvfp4(N, K)
            qa.act_quant(qa.NVFP4, dev(w), q, s, ts, 0,
                         qa.workspace(qa.act_quant_workspace(qa.NVFP4, N, K)))
            w8 = qa.empty_int8_planes(N, K)
            qa.int8_weight_planes(q, s, w8, N, K)
            self.w.append((q, s, ts, w8, N, K))
        # the oracle's encoding of the same weights, checked once
        self.wdeq = []
        for w, (q, s, ts, _, _, _) in zip((wu, wd), self.w):
            oq, os_, ots = Q.nvfp4_encode(w)
            np.testing.assert_array_equal(host(q), oq)
            np.testing.assert_array_equal(host(s), os_)
            assert host(ts)[0] == ots
            self.wdeq.append(Q.nvfp4_decode(oq, os_, ots))
        M, K, F_ = self.M, self.K, self.F
        bf = t.bfloat16
        self.h = t.empty((M, F_), dtype=bf, device="cuda")
        self.y = t.empty((M, K), dtype=bf, device="cuda")
        self.a4 = qa.empty_nvfp4(M, F_)
        self.a8 = qa.empty_int8_act(M, F_)
        self.qws = qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, F_))
        self.gws = qa.workspace(max(qa.qlinear_workspace(f, M, N, K)
                                    for f in (qa.NVFP4, qa.INT8) for (_, _, _, _, N, K) in self.w))
        self.rws = qa.workspace(qa.reduce_workspace(M * K))
        self.sums = t.zeros(2, dtype=t.float64, device="cuda")

    def linear(self, fmt, x, w, y, gelu):
        qa = _qa()
        q, s, ts, w8, N, K = w
        M = self.M
        epi = qa.EPI_GELU_TANH if gelu else qa.EPI_NONE
        if fmt == 0:
            aq = self.a4[0].view(-1)[: M * K // 2].view(M, K // 2)
            asc = self.a4[1].view(-1)[: M * K // 16].view(M, K // 16)
            qa.act_quant(qa.NVFP4, x, aq, asc, self.a4[2], 0, self.qws)
            qa.qlinear_nvfp4(aq, asc, self.a4[2], q, s, ts, y, M, N, K, epi=epi, ws=self.gws)
            return aq, asc, self.a4[2]
        aq = self.a8[0].view(-1)[: M * K].view(M, K)
        qa.act_quant(qa.INT8, x, aq, self.a8[1])
        qa.qlinear_int8(aq, self.a8[1], q, s, ts, y, M, N, K, epi=epi, ws=self.gws, w8=w8)
        return aq, self.a8[1], None

    def step(self, x, fmt, check_rows=None):
        """One FFN residual block step in format fmt (both linears); returns
        (out device tensor, Gamma sums as numpy)."""
        qa, t = _qa(), torch()
        xd = dev(x)
        a_up = self.linear(fmt, xd, self.w[0], self.h, True)
        if check_rows is not None:
            self._check(fmt, x, a_up, self.w[0], self.wdeq[0], self.h, True, check_rows)
        a_dn = self.linear(fmt, self.h.view(t.int16), self.w[1], self.y, False)
        if check_rows is not None:
            self._check(fmt, None, a_dn, self.w[1], self.wdeq[1], self.y, False, check_rows)
        out = t.empty_like(xd)
        qa.tdc_apply(xd, self.y.view(t.int16), out, self.sums, self.rws)
        t.cuda.synchronize()
        return out, host(self.sums)

    def _check(self, fmt, x_host, a, w, wdeq, y, gelu, rows):
        t = torch()
        t.cuda.synchronize()
        if x_host is None:                     # the hidden activation
            x_host = host(self.h)
        K = w[5]
        xr = x_host[rows]
        if fmt == 0:
            ts = Q.nvfp4_tensor_scale(x_host)
            assert host(a[2])[0] == ts
            oc, os_, _ = Q.nvfp4_encode(xr, tscale=ts)
            np.testing.assert_array_equal(host(a[0])[rows], oc)
            np.testing.assert_array_equal(host(a[1])[rows], os_)
            ad = Q.nvfp4_decode(oc, os_, ts)
        else:
            oq, os_ = Q.int8_encode(xr)
            np.testing.assert_array_equal(host(a[0])[rows], oq)
            np.testing.assert_array_equal(host(a[1])[rows], os_)
            ad = Q.int8_decode(oq, os_)
        ref = F.bf16_to_f64(F.f64_to_bf16_rne(G.linear_ref(ad, wdeq, gelu=gelu)))
        got = F.bf16_to_f64(host(y)[rows])
        assert rel_fro(got, ref) <= 1e-3


def test_ffn_config_dmpq_full_size():
    qa = _qa()
    blk = FFNBlock()
    M = blk.M
    rows = sample_rows(M, 48, seed=9)
    alpha = np.full(2, ALPHA, np.float32)
    beta = np.full(2, BETA, np.float32)

    # the drifting inputs x_t, made once for both passes
    xs, x = [], blk.x0
    for t_ in range(STEPS):
        x = synth.drift(3, t_, x)
        xs.append(x)
    # calibration pass: every linear INT8 (the t = 0 choice), Gamma per step
    gam_cal = []
    for t_ in range(STEPS):
        _, s = blk.step(xs[t_], 1)
        gam_cal.append(qa.gamma_from_sums(s))
    # predictions of steps 1..9 (Gamma of steps 0..8), both linears of each
    n = STEPS - 1
    p = T.predictions(np.array(gam_cal[:-1]), np.full(2 * n, ALPHA, np.float32),
                      np.full(2 * n, BETA, np.float32), 2)
    tau = T.tau_for_half(p)
    assert 0.3 <= (p > tau).mean() <= 0.7

    # the DMPQ pass
    gamma_prev = None
    checked_fmt = set()
    masks = []
    for t_ in range(STEPS):
        x = xs[t_]
        mask = qa.dmpq_mask(None if gamma_prev is None else np.array([gamma_prev]), alpha, beta,
                            tau, 1, 2)
        omask = T.dmpq_mask(None if gamma_prev is None else np.array([gamma_prev]), alpha, beta,
                            tau, 2)
        np.testing.assert_array_equal(mask, omask)
        assert mask[0] == mask[1]               # one Gamma per block: one format
        fmt = int(mask[0])
        masks.append(fmt)
        check = t_ < 2 or fmt not in checked_fmt
        out, s = blk.step(x, fmt, rows if check else None)
        if check:
            checked_fmt.add(fmt)
            # residual add bit-exact and the Gamma sums of the whole tensors
            y_rows = host(blk.y)[rows]
            np.testing.assert_array_equal(host(out)[rows],
                                          T.tdc_apply(x[rows].ravel(), y_rows.ravel()).reshape(
                                              len(rows), -1))
            ref = T.gamma_sums(x, host(out), summation="pairwise")
            assert np.all(np.abs(s - ref) <= 1e-12 * np.abs(ref))
        gamma_prev = qa.gamma_from_sums(s)
        print(f"[ffn] step {t_} format {'INT8' if fmt else 'NVFP4'} gamma {gamma_prev:.6f} "
              f"tau {tau:.6f} checked {check}", flush=True)
    assert masks[0] == 1                         # no Gamma at t = 0: INT8
    assert checked_fmt == {0, 1} or len(set(masks[1:])) == 1
