"""Calls that take their operands from a device gate byte (one launch for
either choice): act_quant_routed against act_quant of the chosen format,
tdc_update_ring / tdc_apply_ring against tdc_update / tdc_apply(_amax) on
the chosen ring slot; the outputs of the choices not taken, and everything
for a byte that selects nothing, are left untouched."""
import numpy as np
import pytest

import synth
from tests._gpu import dev, host, torch

pytestmark = pytest.mark.gpu


def _qa():
    import mixed_precision_quantized_act_amd as qa
    return qa


def _byte(v):
    return torch().tensor([v], dtype=torch().uint8, device="cuda")


def _sentinels(M, K):
    qa, t = _qa(), torch()
    q4, s4, ts4 = qa.empty_nvfp4(M, K)
    q8, s8 = qa.empty_int8_act(M, K)
    for b in (q4, s4, q8):
        b.fill_(0x5A)
    ts4.fill_(-7.0)
    s8.fill_(-9.0)
    return q4, s4, ts4, q8, s8


@pytest.mark.parametrize("flags", [0, 1, 2])
@pytest.mark.parametrize("M,K", [(300, 1920), (37, 48), (2, 7680)])
def test_act_quant_routed(M, K, flags):
    qa, t = _qa(), torch()
    x = dev(synth.activations(11, M, K, "t3"))
    ws = qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, K))
    if flags == qa.TSCALE_GIVEN:
        ts_given = 0.0123
    if flags == qa.AMAX_GIVEN:
        # partial maxima as a producer leaves them: those of act_quant's own pass
        ref_ws = qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, K))
        ref_ws.zero_()                               # slots past the pass's workgroups: 0
        rq, rs, rts = qa.empty_nvfp4(M, K)
        qa.act_quant(qa.NVFP4, x, rq, rs, rts, 0, ref_ws)        # fills ref_ws's partial maxima
        t.cuda.synchronize()
        ws[:4096].copy_(ref_ws[:4096])
    # reference outputs of both formats
    r4 = qa.empty_nvfp4(M, K)
    if flags == qa.TSCALE_GIVEN:
        r4[2].fill_(ts_given)
    rws = qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, K))
    if flags == qa.AMAX_GIVEN:
        rws[:4096].copy_(ws[:4096])
    qa.act_quant(qa.NVFP4, x, r4[0], r4[1], r4[2], flags, rws)
    r8 = qa.empty_int8_act(M, K)
    qa.act_quant(qa.INT8, x, r8[0], r8[1])
    t.cuda.synchronize()
    for route in (qa.ROUTE_NVFP4, qa.ROUTE_INT8, 0):
        q4, s4, ts4, q8, s8 = _sentinels(M, K)
        if flags == qa.TSCALE_GIVEN:
            ts4.fill_(ts_given)
        before = [host(b).copy() for b in (q4, s4, ts4, q8, s8)]
        qa.act_quant_routed(_byte(route), x, q4, s4, ts4, flags, ws, q8, s8)
        t.cuda.synchronize()
        got = [host(b) for b in (q4, s4, ts4, q8, s8)]
        want4 = [host(b) for b in r4] if route == qa.ROUTE_NVFP4 else before[:3]
        want8 = [host(b) for b in r8] if route == qa.ROUTE_INT8 else before[3:]
        for g, w in zip(got, want4 + want8):
            np.testing.assert_array_equal(g, w, err_msg=f"route {route} flags {flags}")


def test_tdc_ring_calls():
    qa, t = _qa(), torch()
    n = 17776 * 64
    rng = np.random.default_rng(5)
    bf = lambda s: dev(synth.bf16_bits(rng.standard_normal(n) * s))
    x_in, x_out = bf(1.0), bf(1.0)
    ws = qa.workspace(qa.reduce_workspace(n))
    for byte in (qa.BLK_RUN0, qa.BLK_RUN1, qa.BLK_SKIP0, qa.BLK_SKIP1, 0):
        ring = [bf(0.1), bf(0.1)]
        keep = [host(r).copy() for r in ring]
        # tdc_update_ring against tdc_update on the chosen slots
        s_got = t.full((4,), -1.0, dtype=t.float64, device="cuda")
        qa.tdc_update_ring(_byte(byte), x_in, x_out, ring[0], ring[1], s_got, ws)
        t.cuda.synchronize()
        if byte in (qa.BLK_RUN0, qa.BLK_RUN1):
            last = 0 if byte == qa.BLK_RUN0 else 1
            prev, new = dev(keep[last]), t.empty_like(x_in)
            s_ref = t.zeros(4, dtype=t.float64, device="cuda")
            qa.tdc_update(x_in, x_out, prev, new, s_ref, ws)
            t.cuda.synchronize()
            np.testing.assert_array_equal(host(ring[last ^ 1]), host(new))
            np.testing.assert_array_equal(host(ring[last]), keep[last])
            np.testing.assert_array_equal(host(s_got), host(s_ref))
        else:
            for r, k in zip(ring, keep):
                np.testing.assert_array_equal(host(r), k)
            assert np.all(host(s_got) == -1.0)
        # tdc_apply_ring (with and without the amax) against tdc_apply(_amax)
        for with_amax in (False, True):
            out = t.full_like(x_in, 0x1234)
            s2 = t.full((2,), -1.0, dtype=t.float64, device="cuda")
            amax = t.zeros(1024, dtype=t.int32, device="cuda") if with_amax else None
            qa.tdc_apply_ring(_byte(byte), x_in, ring[0], ring[1], out, s2, ws, out_amax=amax)
            t.cuda.synchronize()
            if byte in (qa.BLK_SKIP0, qa.BLK_SKIP1):
                slot = ring[0 if byte == qa.BLK_SKIP0 else 1]
                ref = t.empty_like(x_in)
                s_ref = t.zeros(2, dtype=t.float64, device="cuda")
                if with_amax:
                    ref_amax = t.zeros(1024, dtype=t.int32, device="cuda")
                    qa.tdc_apply_amax(x_in, slot, ref, ref_amax, s_ref, ws)
                else:
                    qa.tdc_apply(x_in, slot, ref, s_ref, ws)
                t.cuda.synchronize()
                np.testing.assert_array_equal(host(out), host(ref))
                np.testing.assert_array_equal(host(s2), host(s_ref))
                if with_amax:
                    np.testing.assert_array_equal(host(amax), host(ref_amax))
            else:
                assert np.all(host(out) == 0x1234) and np.all(host(s2) == -1.0)
                if with_amax:
                    assert not host(amax).any()


# qlinear_routed against the plain call of the chosen format: small, with
# bias + GELU + the output |max| and ragged N, a K-split last round in both
# formats (only the slices and fixups launch), many tiles with ragged M and
# N in one routed launch (7 units: no persistent INT8 kernel), and many
# short-K tiles, where the INT8 whole tiles take the persistent kernel and
# each format launches on its own
ROUTED_SHAPES = [(300, 256, 384, False, False, False), (300, 200, 192, True, True, True),
                 (600, 704, 3840, False, False, True), (2000, 1000, 448, False, True, True),
                 (4452, 1960, 1920, False, True, False), (4452, 3840, 1920, True, True, True)]


@pytest.mark.parametrize("route", [0, 1, 2, 3])
@pytest.mark.parametrize("M,N,K,bias,gelu,amax", ROUTED_SHAPES)
def test_qlinear_routed(M, N, K, bias, gelu, amax, route):
    qa, t = _qa(), torch()
    x = dev(synth.activations(13, M, K, "normal", 4, 20.0))
    w = dev(synth.weight(13, 0, N, K))
    a4 = qa.empty_nvfp4(M, K)
    qa.act_quant(qa.NVFP4, x, a4[0], a4[1], a4[2], 0,
                 qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, K)))
    a8 = qa.empty_int8_act(M, K)
    qa.act_quant(qa.INT8, x, a8[0], a8[1])
    wq = qa.empty_nvfp4(N, K)
    qa.act_quant(qa.NVFP4, w, wq[0], wq[1], wq[2], 0,
                 qa.workspace(qa.act_quant_workspace(qa.NVFP4, N, K)))
    w8 = qa.empty_int8_planes(N, K)
    assert qa.int8_weight_planes(wq[0], wq[1], w8, N, K) == 0
    b = dev(np.random.default_rng(5).normal(0, 0.5, N).astype(np.float32)).to(t.bfloat16) \
        if bias else None
    epi = qa.EPI_GELU_TANH if gelu else qa.EPI_NONE
    ws = qa.workspace(qa.qlinear_routed_workspace(M, N, K))
    slots = t.zeros(1024, dtype=t.int32, device="cuda")
    # reference: the plain call of the format the byte selects
    ref = t.empty((M, N), dtype=t.bfloat16, device="cuda")
    ref_slots = t.zeros(1024, dtype=t.int32, device="cuda")
    fmt = 1 if route & 1 else (2 if route & 2 else 0)
    if fmt == 1:
        if amax:
            qa.qlinear_nvfp4_amax(a4[0], a4[1], a4[2], wq[0], wq[1], wq[2], ref, ref_slots, M, N, K,
                                  bias=b, epi=epi, ws=ws)
        else:
            qa.qlinear_nvfp4(a4[0], a4[1], a4[2], wq[0], wq[1], wq[2], ref, M, N, K, bias=b,
                             epi=epi, ws=ws)
    elif fmt == 2:
        if amax:
            qa.qlinear_int8_amax(a8[0], a8[1], None, None, wq[2], ref, ref_slots, M, N, K, bias=b,
                                 epi=epi, ws=ws, w8=w8)
        else:
            qa.qlinear_int8(a8[0], a8[1], None, None, wq[2], ref, M, N, K, bias=b, epi=epi, ws=ws,
                            w8=w8)
    t.cuda.synchronize()
    y = t.full((M, N), -3.0, dtype=t.bfloat16, device="cuda")
    qa.qlinear_routed(_byte(route), a4[0], a4[1], a4[2], a8[0], a8[1], wq[0], wq[1], wq[2], w8,
                      y, M, N, K, bias=b, epi=epi, y_amax=slots if amax else None, ws=ws)
    t.cuda.synchronize()
    if fmt == 0:
        assert bool((y == -3.0).all())
        assert int(slots.abs().max()) == 0
        return
    assert t.equal(y.view(t.int16), ref.view(t.int16))
    if amax:
        # the output's |max| (how it spreads over the 1024 words follows the
        # launch's workgroups)
        assert int(slots.max()) == int(ref_slots.max())
        yb = host(y.view(t.int16)).astype(np.uint32) & 0x7FFF
        assert int(slots.max()) == int(yb.max()) << 16


@pytest.mark.parametrize("M,N,K", [(300, 200, 192), (600, 704, 3840), (4452, 1960, 1920)])
def test_qlinear_routed_under_thread_gate(M, N, K):
    # a gate set with qa_set_gate applies to qlinear_routed as to every call:
    # closed, no launch of either format touches y, the |max| words or the
    # workspace's effect (one routed launch; a K split; the persistent INT8
    # kernel); open, the outputs are those of the ungated call
    qa, t = _qa(), torch()
    x = dev(synth.activations(17, M, K, "normal"))
    w = dev(synth.weight(17, 0, N, K))
    a4 = qa.empty_nvfp4(M, K)
    qa.act_quant(qa.NVFP4, x, a4[0], a4[1], a4[2], 0,
                 qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, K)))
    a8 = qa.empty_int8_act(M, K)
    qa.act_quant(qa.INT8, x, a8[0], a8[1])
    wq = qa.empty_nvfp4(N, K)
    qa.act_quant(qa.NVFP4, w, wq[0], wq[1], wq[2], 0,
                 qa.workspace(qa.act_quant_workspace(qa.NVFP4, N, K)))
    w8 = qa.empty_int8_planes(N, K)
    assert qa.int8_weight_planes(wq[0], wq[1], w8, N, K) == 0
    ws = qa.workspace(qa.qlinear_routed_workspace(M, N, K))
    flag = t.zeros(1, dtype=t.uint8, device="cuda")
    for route in (qa.ROUTE_NVFP4, qa.ROUTE_INT8):
        ref = t.empty((M, N), dtype=t.bfloat16, device="cuda")
        ref_slots = t.zeros(1024, dtype=t.int32, device="cuda")
        qa.qlinear_routed(_byte(route), a4[0], a4[1], a4[2], a8[0], a8[1], wq[0], wq[1], wq[2],
                          w8, ref, M, N, K, epi=qa.EPI_GELU_TANH, y_amax=ref_slots, ws=ws)
        for state in (0, 4, 3):                   # closed, closed (other bit), open
            flag.fill_(state)
            y = t.full((M, N), -3.0, dtype=t.bfloat16, device="cuda")
            slots = t.zeros(1024, dtype=t.int32, device="cuda")
            with qa.gate(flag, 3):
                qa.qlinear_routed(_byte(route), a4[0], a4[1], a4[2], a8[0], a8[1], wq[0], wq[1],
                                  wq[2], w8, y, M, N, K, epi=qa.EPI_GELU_TANH, y_amax=slots, ws=ws)
            t.cuda.synchronize()
            if state & 3:
                assert t.equal(y.view(t.int16), ref.view(t.int16)), (route, state)
                assert int(slots.max()) == int(ref_slots.max())
            else:
                assert bool((y == -3.0).all()), (route, state)
                assert int(slots.abs().max()) == 0
