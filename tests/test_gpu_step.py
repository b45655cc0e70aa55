"""Device-side step control: the gate of a call (qa_set_gate) and the
timestep decisions made on the device (qa_decide_step), for a small DiT
stack over 10 drifting steps -- enqueued eagerly, and captured once in a
HIP graph and replayed -- against the same stack driven by the host
decisions (dmpq_mask, tdc_decide).  Every call runs the same kernels on the
same inputs either way, so outputs, masks and skips must agree bit for
bit."""
import math

import numpy as np
import pytest

import synth
from tests._gpu import dev, host, torch

pytestmark = pytest.mark.gpu

L, J, H, F, M = 4, 4, 256, 1024, 500
SHAPES = [(3 * H, H), (H, H), (F, H), (H, F)]


def _qa():
    import mixed_precision_quantized_act_amd as qa
    return qa


def test_gate_closed_leaves_outputs():
    qa, t = _qa(), torch()
    x = dev(synth.activations(1, 300, 256, "normal"))
    w = dev(synth.activations(2, 200, 256, "normal"))
    flag = t.zeros(1, dtype=t.uint8, device="cuda")
    wq, ws, wts = qa.empty_nvfp4(200, 256)
    qa.act_quant(qa.NVFP4, w, wq, ws, wts, 0, qa.workspace(qa.act_quant_workspace(qa.NVFP4, 200, 256)))
    outs = {}
    for state in ("open", "closed", "ungated"):
        flag.fill_(3 if state == "open" else 4)
        aq, asc, ats = qa.empty_nvfp4(300, 256)
        a8, s8 = qa.empty_int8_act(300, 256)
        y = t.empty((300, 200), dtype=t.float32, device="cuda")
        d = t.empty(300 * 256, dtype=t.int16, device="cuda")
        s4 = t.zeros(4, dtype=t.float64, device="cuda")
        for b in (aq, asc, a8, d):
            b.view(t.uint8).fill_(0x5A)
        for b in (ats, s8, y):
            b.fill_(-7.0)
        s4.fill_(-7.0)
        if state != "ungated":
            qa.set_gate(flag, 2)
        try:
            qa.act_quant(qa.NVFP4, x, aq, asc, ats, 0, qa.workspace(qa.act_quant_workspace(qa.NVFP4, 300, 256)))
            qa.act_quant(qa.INT8, x, a8, s8)
            qa.qlinear_int8(a8, s8, wq, ws, wts, y, 300, 200, 256, out=qa.OUT_F32,
                            ws=qa.workspace(qa.qlinear_workspace(qa.INT8, 300, 200, 256)))
            xv = x.view(t.int16).view(-1)
            qa.tdc_update(xv, xv, None, d, s4, qa.workspace(qa.reduce_workspace(xv.numel())))
        finally:
            qa.set_gate(None)
        t.cuda.synchronize()
        outs[state] = [host(b).copy() for b in (aq, asc, ats, a8, s8, y, d, s4)]
    for a, b in zip(outs["open"], outs["ungated"]):
        np.testing.assert_array_equal(a, b)
    closed = outs["closed"]
    for a in (closed[0], closed[1], closed[3], closed[6]):
        assert (a.view(np.uint8) == 0x5A).all()
    for a in (closed[2], closed[4], closed[5], closed[7]):
        assert (a == -7.0).all()


class _Stack:
    """Weights, buffers and both drivers of the small stack."""

    def __init__(self, L=L, H=H, F=F, M=M, seed=31):
        qa, t = _qa(), torch()
        self.qa, self.t = qa, t
        self.L, self.J, self.H, self.F, self.M = L, J, H, F, M
        SHAPES = [(3 * H, H), (H, H), (F, H), (H, F)]
        gen = t.Generator(device="cuda")
        gen.manual_seed(seed)
        qw = qa.workspace(qa.act_quant_workspace(qa.NVFP4, F, F))
        self.layers = []
        for _ in range(L):
            lay = []
            for (N, K) in SHAPES:
                w = (t.randn((N, K), generator=gen, device="cuda") * 0.02).to(t.bfloat16)
                q, sc, ts = qa.empty_nvfp4(N, K)
                qa.act_quant(qa.NVFP4, w.view(t.int16), q, sc, ts, 0, qw)
                w8 = qa.empty_int8_planes(N, K)
                assert qa.int8_weight_planes(q, sc, w8, N, K) == 0
                lay.append((q, sc, ts, N, K, w8))
            self.layers.append(lay)
        bf = t.bfloat16
        self.qkv = t.empty((M, 3 * H), dtype=bf, device="cuda")
        self.o = t.empty((M, H), dtype=bf, device="cuda")
        self.x1 = t.empty((M, H), dtype=bf, device="cuda")
        self.u = t.empty((M, F), dtype=bf, device="cuda")
        self.dd = t.empty((M, H), dtype=bf, device="cuda")
        self.a4 = qa.empty_nvfp4(M, F)
        self.a8 = qa.empty_int8_act(M, F)
        self.qws = qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, F))
        self.gws = qa.workspace(max([qa.qlinear_workspace(f, M, N, K) for f in (qa.NVFP4, qa.INT8)
                                     for (N, K) in SHAPES] +
                                    [qa.qlinear_routed_workspace(M, N, K) for (N, K) in SHAPES]))
        self.rws = qa.workspace(qa.reduce_workspace(M * H))
        self.ring = [[t.zeros((M, H), dtype=bf, device="cuda") for _ in range(2)] for _ in range(L)]
        self.outs = [t.empty((M, H), dtype=bf, device="cuda") for _ in range(L)]
        self.sums = t.zeros((L, 4), dtype=t.float64, device="cuda")
        self.alpha = np.full(L * J, 1.0, np.float32)
        self.beta = np.full(L * J, 0.01, np.float32)
        self.alpha_d, self.beta_d = dev(self.alpha), dev(self.beta)
        self.t_ctr = t.zeros(1, dtype=t.int32, device="cuda")
        self.bstate = t.zeros((L, 4), dtype=t.uint8, device="cuda")
        self.d_prev = t.zeros(L, dtype=t.float64, device="cuda")
        self.blk = t.zeros(L, dtype=t.uint8, device="cuda")
        self.lin = t.zeros(L * J, dtype=t.uint8, device="cuda")
        self.mask_out = t.zeros(L * J, dtype=t.uint8, device="cuda")
        self.skip_out = t.zeros(L, dtype=t.uint8, device="cuda")
        self.x_in = t.empty((M, H), dtype=bf, device="cuda")

    def reset(self):
        for r in self.ring:
            for b in r:
                b.zero_()
        for b in (self.sums, self.t_ctr, self.bstate, self.d_prev):
            b.zero_()

    def linear(self, fmt, x, ldx, lay, y, gelu):
        L, J, H, F, M = self.L, self.J, self.H, self.F, self.M
        qa, t = self.qa, self.t
        q, sc, ts, N, K, w8 = lay
        xv = t.as_strided(x, (M, K), (ldx, 1)).view(t.int16)
        epi = qa.EPI_GELU_TANH if gelu else qa.EPI_NONE
        if fmt == 0:
            aq = self.a4[0].view(-1)[: M * K // 2].view(M, K // 2)
            asc = self.a4[1].view(-1)[: M * K // 16].view(M, K // 16)
            qa.act_quant(qa.NVFP4, xv, aq, asc, self.a4[2], 0, self.qws, M=M, K=K, ldx=ldx)
            qa.qlinear_nvfp4(aq, asc, self.a4[2], q, sc, ts, y, M, N, K, epi=epi, ws=self.gws)
        else:
            aq = self.a8[0].view(-1)[: M * K].view(M, K)
            qa.act_quant(qa.INT8, xv, aq, self.a8[1], M=M, K=K, ldx=ldx)
            qa.qlinear_int8(aq, self.a8[1], q, sc, ts, y, M, N, K, epi=epi, ws=self.gws, w8=w8)

    def gemm(self, fmt, lay, y, gelu, K):
        L, J, H, F, M = self.L, self.J, self.H, self.F, self.M
        qa = self.qa
        q, sc, ts, N, _, w8 = lay
        epi = qa.EPI_GELU_TANH if gelu else qa.EPI_NONE
        if fmt == 0:
            aq = self.a4[0].view(-1)[: M * K // 2].view(M, K // 2)
            asc = self.a4[1].view(-1)[: M * K // 16].view(M, K // 16)
            qa.qlinear_nvfp4(aq, asc, self.a4[2], q, sc, ts, y, M, N, K, epi=epi, ws=self.gws)
        else:
            aq = self.a8[0].view(-1)[: M * K].view(M, K)
            qa.qlinear_int8(aq, self.a8[1], q, sc, ts, y, M, N, K, epi=epi, ws=self.gws, w8=w8)

    def routed_linear(self, flag, x, ldx, lay, y, gelu):
        """One act_quant launch and one GEMM launch in the format the linear's
        flag selects."""
        L, J, H, F, M = self.L, self.J, self.H, self.F, self.M
        qa, t = self.qa, self.t
        K = lay[4]
        xv = t.as_strided(x, (M, K), (ldx, 1)).view(t.int16)
        aq4 = self.a4[0].view(-1)[: M * K // 2].view(M, K // 2)
        as4 = self.a4[1].view(-1)[: M * K // 16].view(M, K // 16)
        aq8 = self.a8[0].view(-1)[: M * K].view(M, K)
        qa.act_quant_routed(flag, xv, aq4, as4, self.a4[2], 0, self.qws, aq8, self.a8[1], M=M,
                            K=K, ldx=ldx)
        q, sc, ts, N, _, w8 = lay
        qa.qlinear_routed(flag, aq4, as4, self.a4[2], aq8, self.a8[1], q, sc, ts, w8, y, M, N, K,
                          epi=qa.EPI_GELU_TANH if gelu else qa.EPI_NONE, ws=self.gws)

    def block(self, l, cur, out, fmts, gated, routed=False):
        """The compute path of block l (linears in formats fmts, or both
        formats gated on the block's linear flags; routed: one act_quant
        launch for both)."""
        L, J, H, F, M = self.L, self.J, self.H, self.F, self.M
        qa, t = self.qa, self.t
        i16 = lambda b: b.view(t.int16)
        lay = self.layers[l]
        ins = [(cur, H, self.qkv, False), (self.qkv.view(-1)[2 * H:], 3 * H, self.o, False),
               (self.x1, H, self.u, True), (self.u, F, self.dd, False)]
        for j, (x, ldx, y, gelu) in enumerate(ins):
            if routed:
                self.routed_linear(self.lin[l * J + j:], x, ldx, lay[j], y, gelu)
            elif gated:
                for fmt, bit in ((0, qa.ROUTE_NVFP4), (1, qa.ROUTE_INT8)):
                    with qa.gate(self.lin[l * J + j:], bit):
                        self.linear(fmt, x, ldx, lay[j], y, gelu)
            else:
                self.linear(fmts[j], x, ldx, lay[j], y, gelu)
            if j == 1:
                if gated:
                    qa.set_gate(self.blk[l:], qa.BLK_RUN0 | qa.BLK_RUN1)
                qa.tdc_apply(i16(cur), i16(self.o), i16(self.x1))
                qa.set_gate(None)
        if gated:
            qa.set_gate(self.blk[l:], qa.BLK_RUN0 | qa.BLK_RUN1)
        qa.tdc_apply(i16(self.x1), i16(self.dd), i16(out))
        qa.set_gate(None)

    def host_run(self, xs, tau, delta):
        """Host decisions, as the benchmark drives the stack."""
        L, J, H, F, M = self.L, self.J, self.H, self.F, self.M
        qa, t = self.qa, self.t
        i16 = lambda b: b.view(t.int16)
        self.reset()
        last, n_stored = [0] * L, [0] * L
        computed_prev = np.zeros(L, np.uint8)
        d_prev = np.full(L, math.inf)
        gamma_prev, rec = None, []
        for step, xd in enumerate(xs):
            if gamma_prev is not None and tau is None:
                p = np.repeat(gamma_prev, J) * self.alpha.astype(np.float64) + self.beta
                srt = np.sort(p)
                tau = 0.5 * (srt[(len(p) - 1) // 2] + srt[len(p) // 2])
            mask = qa.dmpq_mask(gamma_prev, self.alpha, self.beta, tau if tau is not None else 0.0, L, J)
            skip = qa.tdc_decide(step, d_prev, computed_prev, delta)
            cur = xd
            for l in range(L):
                out = self.outs[l]
                if skip[l]:
                    qa.tdc_apply(i16(cur), i16(self.ring[l][last[l]]), i16(out), self.sums[l, :2],
                                 self.rws)
                    computed_prev[l] = 0
                else:
                    self.block(l, cur, out, mask[l * J:(l + 1) * J], False)
                    nxt = last[l] ^ 1
                    qa.tdc_update(i16(cur), i16(out), i16(self.ring[l][last[l]]),
                                  i16(self.ring[l][nxt]), self.sums[l], self.rws)
                    last[l] = nxt
                    n_stored[l] = min(n_stored[l] + 1, 2)
                    computed_prev[l] = 1
                cur = out
            hs = host(self.sums).copy()
            gamma_prev = np.array([qa.gamma_from_sums(hs[l, :2]) for l in range(L)])
            for l in range(L):
                if not skip[l]:
                    d_prev[l] = qa.rel_l2_from_sums(hs[l]) if n_stored[l] > 1 else math.inf
            rec.append((mask.copy(), skip.copy(), host(self.outs[-1]).copy()))
        return rec, tau

    def device_step(self, tau, delta, routed=False):
        """One step, every path enqueued under its gate (routed: the calls
        that take their format or ring slot from the gate byte, one launch
        each)."""
        L, J, H, F, M = self.L, self.J, self.H, self.F, self.M
        qa, t = self.qa, self.t
        i16 = lambda b: b.view(t.int16)
        qa.decide_step(self.sums, self.alpha_d, self.beta_d, tau, delta, L, J, self.t_ctr,
                       self.bstate, self.d_prev, self.blk, self.lin, self.mask_out, self.skip_out)
        cur = self.x_in
        for l in range(L):
            out = self.outs[l]
            r0, r1 = self.ring[l]
            if routed:
                qa.tdc_apply_ring(self.blk[l:], i16(cur), i16(r0), i16(r1), i16(out),
                                  self.sums[l, :2], self.rws)
            else:
                for slot, bit in ((r0, qa.BLK_SKIP0), (r1, qa.BLK_SKIP1)):
                    with qa.gate(self.blk[l:], bit):
                        qa.tdc_apply(i16(cur), i16(slot), i16(out), self.sums[l, :2], self.rws)
            self.block(l, cur, out, None, True, routed)
            if routed:
                qa.tdc_update_ring(self.blk[l:], i16(cur), i16(out), i16(r0), i16(r1),
                                   self.sums[l], self.rws)
            else:
                for prev, nxt, bit in ((r0, r1, qa.BLK_RUN0), (r1, r0, qa.BLK_RUN1)):
                    with qa.gate(self.blk[l:], bit):
                        qa.tdc_update(i16(cur), i16(out), i16(prev), i16(nxt), self.sums[l],
                                      self.rws)
            cur = out


def _inputs(M=M, H=H, steps=10):
    x = synth.activations(1, M, H, "normal")
    xs = []
    for step in range(steps):
        x = synth.drift(1, step, x)
        xs.append(dev(x).view(torch().bfloat16))
    return xs


@pytest.mark.parametrize("routed", [False, True])
@pytest.mark.parametrize("delta", [10.0, 0.05, 0.0])
def test_device_decisions_eager_and_graph(delta, routed):
    # delta 10: every block that ran at t-1 is skipped from t = 2 on (both
    # paths, both ring slots); 0.05: the pages' threshold, some blocks;
    # 0: nothing is skipped
    t = torch()
    st = _Stack()
    xs = _inputs()
    ref, tau = st.host_run(xs, None, delta)
    skips = np.array([r[1] for r in ref])
    if delta > 1:
        assert skips[2:].sum() >= L * 4 and not skips[:2].any()
    if delta == 0.0:
        assert not skips.any()
    assert 0 < sum(r[0].sum() for r in ref[1:]) < 9 * L * J      # both formats occur

    st.reset()
    for step, xd in enumerate(xs):
        st.x_in.copy_(xd)
        st.device_step(tau, delta, routed)
        t.cuda.synchronize()
        np.testing.assert_array_equal(host(st.mask_out), ref[step][0], err_msg=f"mask, step {step}")
        np.testing.assert_array_equal(host(st.skip_out), ref[step][1], err_msg=f"skip, step {step}")
        np.testing.assert_array_equal(host(st.outs[-1]), ref[step][2], err_msg=f"output, step {step}")

    # captured once, replayed per step with the input copied in between
    st.reset()
    g = t.cuda.CUDAGraph()
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):
        with t.cuda.graph(g, stream=s):
            st.device_step(tau, delta, routed)
    t.cuda.current_stream().wait_stream(s)
    st.reset()
    t.cuda.synchronize()
    for step, xd in enumerate(xs):
        st.x_in.copy_(xd)
        g.replay()
        t.cuda.synchronize()
        np.testing.assert_array_equal(host(st.mask_out), ref[step][0], err_msg=f"graph mask, step {step}")
        np.testing.assert_array_equal(host(st.skip_out), ref[step][1], err_msg=f"graph skip, step {step}")
        np.testing.assert_array_equal(host(st.outs[-1]), ref[step][2], err_msg=f"graph output, step {step}")


def test_device_decisions_full_width_graph():
    # the same at the CogVideoX-2B block width (17776 tokens, H 1920, FFN
    # 7680): two blocks over five steps, routed calls captured once and
    # replayed, against host decisions bit for bit; the routed GEMM takes
    # its persistent-INT8 path (QKV, up), its one-launch path and K splits
    # (down), the NVFP4 scale re-layout; delta 10 skips blocks from t = 2
    t = torch()
    st = _Stack(L=2, H=1920, F=7680, M=17776, seed=7)
    xs = _inputs(17776, 1920, 5)
    ref, tau = st.host_run(xs, None, 10.0)
    skips = np.array([r[1] for r in ref])
    assert skips[2:].any() and not skips[:2].any()
    masks = np.array([r[0] for r in ref[1:]])
    assert 0 < masks.sum() < masks.size                 # both formats occur
    st.reset()
    g = t.cuda.CUDAGraph()
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):
        with t.cuda.graph(g, stream=s):
            st.device_step(tau, 10.0, routed=True)
    t.cuda.current_stream().wait_stream(s)
    st.reset()
    t.cuda.synchronize()
    for step, xd in enumerate(xs):
        st.x_in.copy_(xd)
        g.replay()
        t.cuda.synchronize()
        np.testing.assert_array_equal(host(st.mask_out), ref[step][0], err_msg=f"mask, step {step}")
        np.testing.assert_array_equal(host(st.skip_out), ref[step][1], err_msg=f"skip, step {step}")
        assert np.array_equal(host(st.outs[-1]), ref[step][2]), f"output, step {step}"


def test_decide_step_against_oracle_rules():
    # qa_decide_step over 7 steps on sums set by hand (zero denominators,
    # a prediction equal to tau, a distance equal to delta), against the
    # oracle's rules driven by the host loop's state update
    from oracle import tdc as T
    qa, t = _qa(), torch()
    L_, J_ = 6, 4
    alpha = np.array([1.0, 2.0, 0.5, 1.0] * L_, np.float32)
    beta = np.array([2.0 ** -7, 0.0, 0.1, -0.2] * L_, np.float32)
    tau, delta = 0.2578125, 0.25          # Gamma 0.25: 0.25 + 2^-7 = tau (a tie)
    rng = np.random.default_rng(4)
    # per step, per block: (S1, S2, S3, S4)
    special = [(1.0, 4.0, 1.0 / 16, 1.0),     # Gamma 0.25, d 0.25 = delta (not below)
               (0.0, 0.0, 0.0, 0.0),          # Gamma 0/0 = 0, d 0/0 = 0
               (3.0, 0.0, 2.0, 0.0),          # Gamma x/0 = inf, d x/0 = inf
               (0.5, 4.0, 1.0 / 64, 1.0)]     # Gamma 0.125, d 0.125
    steps = 7
    sums_seq = []
    for s_ in range(steps):
        rows = []
        for l in range(L_):
            if (l + s_) % 3 == 0:
                rows.append(special[(l + s_) % 4])
            else:
                rows.append(tuple(float(v) for v in rng.uniform(0.0, 1.0, 4)))
        sums_seq.append(np.array(rows, np.float64))
    sums = t.zeros((L_, 4), dtype=t.float64, device="cuda")
    t_ctr = t.zeros(1, dtype=t.int32, device="cuda")
    bstate = t.zeros((L_, 4), dtype=t.uint8, device="cuda")
    d_prev = t.zeros(L_, dtype=t.float64, device="cuda")
    blk = t.zeros(L_, dtype=t.uint8, device="cuda")
    lin = t.zeros(L_ * J_, dtype=t.uint8, device="cuda")
    mask_o = t.zeros(L_ * J_, dtype=t.uint8, device="cuda")
    skip_o = t.zeros(L_, dtype=t.uint8, device="cuda")
    # the host loop's state
    computed = np.zeros(L_, bool)
    n_st = np.zeros(L_, int)
    last = np.zeros(L_, int)
    dp = np.full(L_, math.inf)
    gamma_prev = None
    for step in range(steps):
        qa.decide_step(sums, dev(alpha), dev(beta), tau, delta, L_, J_, t_ctr, bstate, d_prev,
                       blk, lin, mask_o, skip_o)
        t.cuda.synchronize()
        if step >= 1:
            prev = sums_seq[step - 1]
            gamma_prev = np.array([T.ratio(prev[l, 0], prev[l, 1]) for l in range(L_)])
            for l in range(L_):
                if computed[l]:
                    last[l] ^= 1
                    n_st[l] = min(n_st[l] + 1, 2)
                    dp[l] = T.rel_l2(prev[l, 2], prev[l, 3]) if n_st[l] >= 2 else math.inf
        mask = T.dmpq_mask(gamma_prev, alpha, beta, tau, J_)
        skip = T.tdc_decide(step, dp, computed, delta)
        np.testing.assert_array_equal(host(mask_o), mask, err_msg=f"mask, step {step}")
        np.testing.assert_array_equal(host(skip_o), skip, err_msg=f"skip, step {step}")
        want_lin = np.where(np.repeat(skip, J_) == 1, 0, np.where(mask == 1, 2, 1))
        np.testing.assert_array_equal(host(lin), want_lin.astype(np.uint8))
        want_blk = np.where(skip == 1, np.where(last == 1, 8, 4), np.where(last == 1, 2, 1))
        np.testing.assert_array_equal(host(blk), want_blk.astype(np.uint8))
        np.testing.assert_array_equal(host(d_prev)[computed | (n_st > 0)],
                                      dp[computed | (n_st > 0)])
        computed = skip == 0
        sums.copy_(t.from_numpy(sums_seq[step]))
    assert int(host(t_ctr)[0]) == steps


def test_gate_closed_k_split_nvfp4_and_amax_calls():
    # a closed gate also stops the NVFP4 GEMM's scale re-layout, the K-split
    # slice and fixup launches, the amax epilogue and tdc_apply_amax
    qa, t = _qa(), torch()
    M, N, K = 600, 704, 3840                       # 9 tiles split in 4 slices
    x = dev(synth.activations(3, M, K, "normal"))
    w = dev(synth.activations(4, N, K, "normal"))
    wq, ws, wts = qa.empty_nvfp4(N, K)
    aq, asc, ats = qa.empty_nvfp4(M, K)
    qw = qa.workspace(qa.act_quant_workspace(qa.NVFP4, max(M, N), K))
    qa.act_quant(qa.NVFP4, w, wq, ws, wts, 0, qw)
    qa.act_quant(qa.NVFP4, x, aq, asc, ats, 0, qw)
    flag = t.zeros(1, dtype=t.uint8, device="cuda")
    gws = qa.workspace(qa.qlinear_workspace(qa.NVFP4, M, N, K))
    y = t.full((M, N), -7.0, dtype=t.bfloat16, device="cuda")
    amax = t.full((1024,), 5, dtype=t.int32, device="cuda")
    d = t.full((M * N,), 0x5A5A, dtype=t.int16, device="cuda")
    am2 = t.full((1024,), 5, dtype=t.int32, device="cuda")
    with qa.gate(flag, 1):
        qa.qlinear_nvfp4(aq, asc, ats, wq, ws, wts, y, M, N, K, ws=gws)
        qa.qlinear_nvfp4_amax(aq, asc, ats, wq, ws, wts, y, amax, M, N, K, ws=gws)
        yv = y.view(t.int16).view(-1)
        qa.tdc_apply_amax(yv, yv, d, am2)
    t.cuda.synchronize()
    assert (host(y).view(np.uint16) == np.uint16(0xC0E0)).all()      # bf16 -7.0
    assert (host(amax) == 5).all() and (host(am2) == 5).all()
    assert (host(d).view(np.uint16) == 0x5A5A).all()
    # and open, the same calls run
    flag.fill_(1)
    with qa.gate(flag, 1):
        qa.qlinear_nvfp4(aq, asc, ats, wq, ws, wts, y, M, N, K, ws=gws)
    t.cuda.synchronize()
    assert not (host(y).view(np.uint16) == np.uint16(0xC0E0)).all()
