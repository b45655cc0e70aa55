"""A synthetic DiT stack driven through libqact, checked against the oracle.

Each block uses the four internal linears of a CogVideoX-style block
(QKV: H -> 3H, O: H -> H, up: H -> F with GELU-tanh, down: F -> H), each
quantized per step to NVFP4 or INT8 by the DMPQ rule, and the Temporal
Delta Cache decides per block whether to compute or reuse its residual.
Attention and normalisation are not part of the quantized-linear path;
the block below keeps the four linear shapes and replaces attention by its
value projection (no token mixing):

    v   = QKV(x)[:, 2H:3H]
    x1  = x + O(v)                       (bf16 residual add: tdc_apply)
    out = x1 + Down(GELU(Up(x1)))        (tdc_apply)

Weights are drawn on the GPU by torch's seeded generator (N(0, 0.02^2),
rounded to bf16 by torch) and quantized to NVFP4 by the library; the
oracle reads the same bf16 bytes back.  Checks are teacher-forced: at every
checked (step, block) the oracle applies its rules to the GPU's own input
tensors and decision inputs.
"""
import math

import numpy as np

from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q
from oracle import tdc as T
from tests._gpu import host, rel_fro, torch

J = 4   # linears per block: QKV, O, up, down


def _qa():
    import mixed_precision_quantized_act_amd as qa
    return qa


class Linear:
    """One NVFP4 weight [N, K] on the GPU (codes, scales, tensor scale) and
    its int8 digit planes for the INT8 path's integer kernel."""

    def __init__(self, w_bf16, keep_bf16=False):
        qa, t = _qa(), torch()
        N, K = w_bf16.shape
        self.N, self.K = N, K
        self.q, self.s, self.ts = qa.empty_nvfp4(N, K)
        ws = qa.workspace(qa.act_quant_workspace(qa.NVFP4, N, K))
        qa.act_quant(qa.NVFP4, w_bf16, self.q, self.s, self.ts, 0, ws)
        self.w8 = qa.empty_int8_planes(N, K)
        qa.int8_weight_planes(self.q, self.s, self.w8, N, K)
        self.w_bf16 = w_bf16 if keep_bf16 else None
        self._deq = None

    def deq(self):
        """Oracle dequantization of the GPU's weight codes (cached)."""
        if self._deq is None:
            self._deq = Q.nvfp4_decode(host(self.q), host(self.s), host(self.ts)[0])
        return self._deq


class Stack:
    def __init__(self, L, H, F_, M, seed, check_blocks=(), rows=48, alpha=1.0, beta=0.01,
                 delta=0.05):
        qa, t = _qa(), torch()
        self.L, self.H, self.F, self.M = L, H, F_, M
        self.alpha = np.full(L * J, alpha, np.float32)
        self.beta = np.full(L * J, beta, np.float32)
        self.delta = delta
        self.check_blocks = set(check_blocks)
        self.rows = np.unique(np.concatenate([
            np.random.default_rng(seed).choice(M, min(rows, M), replace=False),
            [0, M - 1]]))
        gen = t.Generator(device="cuda")
        gen.manual_seed(seed)
        shapes = [(3 * H, H), (H, H), (F_, H), (H, F_)]
        self.layers = []
        for l in range(L):
            lay = []
            for (N, K) in shapes:
                w = (t.randn((N, K), generator=gen, device="cuda", dtype=t.float32) * 0.02)
                lay.append(Linear(w.to(t.bfloat16), keep_bf16=l in self.check_blocks))
            self.layers.append(lay)
        dev = "cuda"
        bf = t.bfloat16
        self.qkv = t.empty((M, 3 * H), dtype=bf, device=dev)
        self.o = t.empty((M, H), dtype=bf, device=dev)
        self.x1 = t.empty((M, H), dtype=bf, device=dev)
        self.u = t.empty((M, F_), dtype=bf, device=dev)
        self.d = t.empty((M, H), dtype=bf, device=dev)
        Kmax = max(H, F_)
        self.a4 = qa.empty_nvfp4(M, Kmax)
        self.a8 = qa.empty_int8_act(M, Kmax)
        self.qws = qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, Kmax))
        self.gws = qa.workspace(max(qa.qlinear_workspace(f, M, N, K)
                                    for f in (qa.NVFP4, qa.INT8) for (N, K) in shapes))
        self.rws = qa.workspace(qa.reduce_workspace(M * H))
        self.ring = [[t.empty((M, H), dtype=bf, device=dev) for _ in range(2)] for _ in range(L)]
        self.last = [1] * L
        self.n_stored = [0] * L
        self.computed_prev = np.zeros(L, np.uint8)
        self.d_prev = np.full(L, math.inf)
        self.gamma_prev = None
        self.tau = None
        self.sums = t.zeros((L, 4), dtype=t.float64, device=dev)
        self.caches = [T.BlockCache(summation="pairwise") for _ in range(L)]  # oracle state
        self.pattern = []
        self.masks = []
        self.checked = 0

    # ------------------------------------------------------------ linears --
    def linear(self, fmt, x, ldx, lay, y, gelu, check):
        """act_quant(fmt) of x [M, K] (row stride ldx) then qlinear -> y."""
        qa, t = _qa(), torch()
        M, K, N = self.M, lay.K, lay.N
        xv = t.as_strided(x, (M, K), (ldx, 1))
        if fmt == 0:
            ats = self.a4[2]
            aq = self.a4[0].view(-1)[: M * K // 2].view(M, K // 2)
            asc = self.a4[1].view(-1)[: M * K // 16].view(M, K // 16)
            qa.act_quant(qa.NVFP4, xv, aq, asc, ats, 0, self.qws, M=M, K=K, ldx=ldx)
            qa.qlinear_nvfp4(aq, asc, ats, lay.q, lay.s, lay.ts, y, M, N, K,
                             epi=qa.EPI_GELU_TANH if gelu else qa.EPI_NONE, ws=self.gws)
        else:
            a8 = self.a8[0].view(-1)[: M * K].view(M, K)
            s8 = self.a8[1]
            qa.act_quant(qa.INT8, xv, a8, s8, M=M, K=K, ldx=ldx)
            qa.qlinear_int8(a8, s8, lay.q, lay.s, lay.ts, y, M, N, K,
                            epi=qa.EPI_GELU_TANH if gelu else qa.EPI_NONE, ws=self.gws, w8=lay.w8)
        if check:
            self._check_linear(fmt, xv, lay, y, gelu)

    def _check_linear(self, fmt, xv, lay, y, gelu):
        t = torch()
        t.cuda.synchronize()
        rows = self.rows
        x_rows = host(xv[rows].contiguous())
        if fmt == 0:
            xs = host(xv.contiguous())
            ts = Q.nvfp4_tensor_scale(xs)
            assert host(self.a4[2])[0] == ts
            K = lay.K
            oc, os_, _ = Q.nvfp4_encode(x_rows, tscale=ts)
            gq = host(self.a4[0].view(-1)[: self.M * K // 2].view(self.M, K // 2)[rows].contiguous())
            gs = host(self.a4[1].view(-1)[: self.M * K // 16].view(self.M, K // 16)[rows].contiguous())
            np.testing.assert_array_equal(gq, oc)
            np.testing.assert_array_equal(gs, os_)
            a_deq = Q.nvfp4_decode(oc, os_, ts)
        else:
            oq, os_ = Q.int8_encode(x_rows)
            K = lay.K
            gq = host(self.a8[0].view(-1)[: self.M * K].view(self.M, K)[rows].contiguous())
            np.testing.assert_array_equal(gq, oq)
            np.testing.assert_array_equal(host(self.a8[1])[rows], os_)
            a_deq = Q.int8_decode(oq, os_)
        ref = G.linear_ref(a_deq, lay.deq(), gelu=gelu)
        got = F.bf16_to_f64(host(y[rows].contiguous()))
        err = rel_fro(got, F.bf16_to_f64(F.f64_to_bf16_rne(ref)))
        assert err <= 1e-3, err
        self.checked += 1

    def check_weights(self, l):
        """GPU weight codes of block l equal the oracle's on sampled rows."""
        for lay in self.layers[l]:
            wb = host(lay.w_bf16)
            ts = Q.nvfp4_tensor_scale(wb)
            assert host(lay.ts)[0] == ts
            r = np.unique(np.concatenate([self.rows % lay.N, [lay.N - 1]]))
            oc, os_, _ = Q.nvfp4_encode(wb[r], tscale=ts)
            np.testing.assert_array_equal(host(lay.q)[r], oc)
            np.testing.assert_array_equal(host(lay.s)[r], os_)
            lay.w_bf16 = None

    # --------------------------------------------------------------- step --
    def step(self, t_, x):
        """One timestep over all blocks; x: bf16 [M, H] device tensor (the
        stack input).  Returns the stack output."""
        qa, t = _qa(), torch()
        L, H = self.L, self.H
        # host decisions from the previous step's sums (one sync per step)
        mask = qa.dmpq_mask(self.gamma_prev, self.alpha, self.beta,
                            self.tau if self.tau is not None else 0.0, L, J)
        if self.gamma_prev is not None and self.tau is None:
            self.tau = T.tau_for_half(T.predictions(self.gamma_prev, self.alpha, self.beta, J))
            mask = qa.dmpq_mask(self.gamma_prev, self.alpha, self.beta, self.tau, L, J)
        omask = T.dmpq_mask(self.gamma_prev, self.alpha, self.beta,
                            self.tau if self.tau is not None else 0.0, J)
        np.testing.assert_array_equal(mask, omask)
        skip = qa.tdc_decide(t_, self.d_prev, self.computed_prev, self.delta)
        oskip = T.tdc_decide(t_, [c.d_prev for c in self.caches],
                             [c.computed_prev for c in self.caches], self.delta)
        np.testing.assert_array_equal(skip, oskip)
        self.masks.append(mask.copy())
        self.pattern.append("".join("S" if s else "C" for s in skip))

        cur = x
        for l in range(L):
            lay = self.layers[l]
            check = l in self.check_blocks
            out = t.empty_like(cur)
            sums = self.sums[l]
            if skip[l]:
                delta = self.ring[l][self.last[l]]
                qa.tdc_apply(cur, delta, out, sums[:2], self.rws)
                if check:
                    t.cuda.synchronize()
                    xin = host(cur)
                    oout = self.caches[l].skip_output(xin)
                    np.testing.assert_array_equal(host(out)[self.rows], oout[self.rows])
                    s_ref = T.gamma_sums(xin, oout, summation="pairwise")
                    _close(host(sums[:2]), s_ref)
                else:
                    self.caches[l].computed_prev = False
                self.computed_prev[l] = 0
            else:
                m = mask[l * J:(l + 1) * J]
                self.linear(m[0], cur, H, lay[0], self.qkv, False, check)
                vslice = self.qkv.view(-1)[2 * H:]
                self.linear(m[1], vslice, 3 * H, lay[1], self.o, False, check)
                qa.tdc_apply(cur, self.o, self.x1)
                self.linear(m[2], self.x1, H, lay[2], self.u, True, check)
                self.linear(m[3], self.u, self.F, lay[3], self.d, False, check)
                qa.tdc_apply(self.x1, self.d, out)
                prev = self.ring[l][self.last[l]] if self.n_stored[l] else None
                nxt = self.last[l] ^ 1
                qa.tdc_update(cur, out, prev, self.ring[l][nxt], sums, self.rws)
                if check:
                    t.cuda.synchronize()
                    xin, xout = host(cur), host(out)
                    dn, s_ref, _ = self.caches[l].computed(xin, xout)
                    np.testing.assert_array_equal(host(self.ring[l][nxt])[self.rows],
                                                  dn[self.rows])
                    _close(host(sums), s_ref)
                self.last[l] = nxt
                self.n_stored[l] = min(self.n_stored[l] + 1, 2)
                self.computed_prev[l] = 1
            cur = out
        hs = host(self.sums)
        gam = np.array([qa.gamma_from_sums(hs[l, :2]) for l in range(L)])
        for l in range(L):
            if not skip[l]:
                d = qa.rel_l2_from_sums(hs[l]) if self.n_stored[l] > 1 else math.inf
                self.d_prev[l] = d
                c = self.caches[l]
                if l not in self.check_blocks:
                    c.d_prev = d            # teacher forcing: the GPU's d
                    c.computed_prev = True
                else:
                    # the oracle's own d for a checked block, within the sum tolerance
                    assert (math.isinf(d) and math.isinf(c.d_prev)) or abs(d - c.d_prev) <= 1e-9 * max(d, 1e-300)
                    c.d_prev = d
        self.gamma_prev = gam
        return cur


def _close(a, b, rtol=1e-12):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert np.all(np.abs(a - b) <= rtol * np.abs(b) + 1e-300), (a, b)
