"""GPU parity of block_gamma, tdc_update and tdc_apply: Delta and applied
outputs bit-exact; sums within 1e-12 relative of the oracle's correctly
rounded sums (the two differ only in summation order)."""
import math

import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import tdc as T
from tests._gpu import dev, host, torch

pytestmark = pytest.mark.gpu


def _qa():
    import mixed_precision_quantized_act_amd as qa
    return qa


def _close(a, b, rtol=1e-12):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert np.all(np.abs(a - b) <= rtol * np.abs(b) + 1e-300), (a, b)


def pair(n, seed, scale=0.1):
    x = synth.bf16_bits(np.random.default_rng(seed).standard_normal(n))
    y = synth.bf16_bits(F.bf16_to_f64(x) + scale * np.random.default_rng(seed + 1).standard_normal(n))
    return x, y


def gpu_gamma(x, y):
    qa, t = _qa(), torch()
    sums = t.zeros(2, dtype=t.float64, device="cuda")
    ws = qa.workspace(qa.reduce_workspace(len(x)))
    qa.block_gamma(dev(x), dev(y), sums, ws)
    t.cuda.synchronize()
    return host(sums)


def gpu_update(x, y, prev):
    qa, t = _qa(), torch()
    n = len(x)
    sums = t.zeros(4, dtype=t.float64, device="cuda")
    dn = t.empty(n, dtype=t.int16, device="cuda")
    ws = qa.workspace(qa.reduce_workspace(n))
    qa.tdc_update(dev(x), dev(y), None if prev is None else dev(prev), dn, sums, ws)
    t.cuda.synchronize()
    return host(dn), host(sums)


def gpu_apply(x, d, with_sums=True, in_place=False):
    qa, t = _qa(), torch()
    n = len(x)
    xd = dev(x)
    out = xd if in_place else t.empty(n, dtype=t.int16, device="cuda")
    sums = t.zeros(2, dtype=t.float64, device="cuda") if with_sums else None
    ws = qa.workspace(qa.reduce_workspace(n)) if with_sums else None
    qa.tdc_apply(xd, dev(d), out, sums, ws)
    t.cuda.synchronize()
    return host(out), (host(sums) if with_sums else None)


@pytest.mark.parametrize("n", [65536, 8, 13, 1, 1000003, 17776 * 1920])
def test_gamma(n):
    x, y = pair(n, 1)
    _close(gpu_gamma(x, y), T.gamma_sums(x, y))


def test_gamma_worked_example():
    x = F.f64_to_bf16_rne(np.array([1, -2, 3, -2], float))
    y = F.f64_to_bf16_rne(np.array([1.5, -2, 3.5, -2], float))
    s = gpu_gamma(x, y)
    assert s.tolist() == [1.0, 8.0]
    qa = _qa()
    assert qa.gamma_from_sums(s) == 0.125


@pytest.mark.parametrize("n", [4096, 21, 17776 * 1920])
@pytest.mark.parametrize("with_prev", [False, True])
def test_update(n, with_prev):
    x, y = pair(n, 2)
    prev = pair(n, 7, scale=0.1)[1] if with_prev else None
    dn, sums = gpu_update(x, y, prev)
    odn, osums = T.tdc_update(x, y, prev)
    np.testing.assert_array_equal(dn, odn)
    _close(sums, osums)


def test_update_rounding_cases():
    x = F.f64_to_bf16_rne(np.array([1.0, 0.0, 3.0, -1e-3, 1e20, 1e-20, 0.0, 1.0]))
    y = F.f64_to_bf16_rne(np.array([300.0, -0.0, 3.0, 1e-3, 1.0, 1e20, 5.0, 1.0]))
    dn, sums = gpu_update(x, y, None)
    odn, osums = T.tdc_update(x, y, None)
    np.testing.assert_array_equal(dn, odn)
    _close(sums, osums)


@pytest.mark.parametrize("n", [4096, 19, 17776 * 1920])
def test_apply(n):
    x, d = pair(n, 3, scale=1.0)
    out, sums = gpu_apply(x, d)
    oout = T.tdc_apply(x, d)
    np.testing.assert_array_equal(out, oout)
    _close(sums, T.gamma_sums(x, oout))
    out2, none = gpu_apply(x, d, with_sums=False, in_place=True)
    assert none is None
    np.testing.assert_array_equal(out2, oout)


def test_apply_worked_ties():
    x = F.f64_to_bf16_rne(np.array([1.0, 256.0] * 8))
    d = F.f64_to_bf16_rne(np.array([2.0 ** -8, 1.0] * 8))
    out, _ = gpu_apply(x, d)
    assert F.bf16_to_f64(out).tolist() == [1.0, 256.0] * 8


def test_relative_l2_worked_example():
    older = F.f64_to_bf16_rne(np.array([1, 2, -1, .5] * 4))
    newer = F.f64_to_bf16_rne(np.array([1.03125, 2.0625, -1.03125, 0.515625] * 4))
    dn, sums = gpu_update(np.zeros(16, np.uint16), newer, older)
    np.testing.assert_array_equal(dn, newer)
    assert _qa().rel_l2_from_sums(sums) == 0.03125


def test_block_cache_teacher_forced():
    # a block driven over 10 drifting steps through the GPU kernels; at
    # every step the oracle state machine sees the same tensors and must
    # agree on the decision, Delta, the applied output and the sums
    qa, t = _qa(), torch()
    n = 4096 * 3
    rng = np.random.default_rng(5)
    base = rng.standard_normal(n)
    x = synth.bf16_bits(rng.standard_normal(n))
    cache = T.BlockCache()
    ring = [t.empty(n, dtype=t.int16, device="cuda") for _ in range(2)]
    last, n_stored, computed_prev, d_prev = 1, 0, False, math.inf
    ws = qa.workspace(qa.reduce_workspace(n))
    pattern = []
    for step in range(10):
        x = synth.drift(4, step, x)
        skip = qa.tdc_decide(step, [d_prev], [computed_prev], 0.05)[0]
        oskip = T.tdc_decide(step, [cache.d_prev], [cache.computed_prev], 0.05)[0]
        assert skip == oskip
        if skip:
            out = t.empty(n, dtype=t.int16, device="cuda")
            sums = t.zeros(2, dtype=t.float64, device="cuda")
            qa.tdc_apply(dev(x), ring[last], out, sums, ws)
            t.cuda.synchronize()
            oout = cache.skip_output(x)
            np.testing.assert_array_equal(host(out), oout)
            _close(host(sums), T.gamma_sums(x, oout))
            computed_prev = False
            pattern.append("S")
        else:
            y = synth.bf16_bits(F.bf16_to_f64(x) + base * (1.0 + 0.01 * step))
            sums = t.zeros(4, dtype=t.float64, device="cuda")
            nxt = last ^ 1
            qa.tdc_update(dev(x), dev(y), ring[last] if n_stored else None, ring[nxt], sums, ws)
            t.cuda.synchronize()
            s = host(sums)
            odn, osums, od = cache.computed(x, y)
            np.testing.assert_array_equal(host(ring[nxt]), odn)
            _close(s, osums)
            d_prev = qa.rel_l2_from_sums(s) if n_stored else math.inf
            if n_stored:
                _close([d_prev], [od])
            last, n_stored, computed_prev = nxt, min(n_stored + 1, 2), True
            pattern.append("C")
    assert "S" in pattern and pattern[:2] == ["C", "C"]


def gpu_rel_err(q, r):
    qa, t = _qa(), torch()
    sums = t.zeros(2, dtype=t.float64, device="cuda")
    ws = qa.workspace(qa.reduce_workspace(len(q)))
    qa.rel_err(dev(q), dev(r), sums, ws)
    t.cuda.synchronize()
    return host(sums)


@pytest.mark.parametrize("n", [65536, 8, 13, 1, 1000003, 17776 * 1920])
def test_rel_err(n):
    r, q = pair(n, seed=31, scale=0.02)
    got = gpu_rel_err(q, r)
    want = T.rel_err_sums(q, r) if n <= 1000003 else (
        T._psum((F.bf16_to_f64(q) - F.bf16_to_f64(r)) ** 2), T._psum(F.bf16_to_f64(r) ** 2))
    _close(got, want)
    qa = _qa()
    e = qa.rel_err_from_sums(got)
    assert abs(e - T.rel_err(*want)) <= 1e-12 * T.rel_err(*want)


def test_rel_err_worked_example():
    r = F.f64_to_bf16_rne(np.array([3.0, 4.0] + [0.0] * 14))
    q = F.f64_to_bf16_rne(np.array([3.0, 5.0] + [0.0] * 14))
    got = gpu_rel_err(q, r)
    assert list(got) == [1.0, 25.0]
    assert _qa().rel_err_from_sums(got) == 0.2


def gpu_cosine(a, b):
    qa, t = _qa(), torch()
    sums = t.zeros(3, dtype=t.float64, device="cuda")
    ws = qa.workspace(qa.reduce_workspace(len(a)))
    qa.delta_cosine(dev(a), dev(b), sums, ws)
    t.cuda.synchronize()
    return host(sums)


@pytest.mark.parametrize("n", [65536, 8, 13, 1, 1000003])
def test_delta_cosine(n):
    a, b = pair(n, seed=37, scale=0.2)
    got = gpu_cosine(a, b)
    want = T.cosine_sums(a, b)
    _close(got, want)
    qa = _qa()
    assert abs(qa.cosine_from_sums(got) - T.cosine(*want)) <= 1e-12


def test_delta_cosine_worked_example():
    v = F.f64_to_bf16_rne(np.array([3.0, 4.0] + [0.0] * 14))
    e1 = F.f64_to_bf16_rne(np.array([1.0] + [0.0] * 15))
    got = gpu_cosine(e1, v)
    assert list(got) == [3.0, 1.0, 25.0]
    assert _qa().cosine_from_sums(got) == 0.6


def test_tdc_apply_amax_feeds_nvfp4_quant():
    # tdc_apply_amax writes the same output and sums as tdc_apply and the
    # |max| of the output; act_quant NVFP4 with that amax (QA_AMAX_GIVEN)
    # equals act_quant's own amax pass and the oracle's encoding
    import mixed_precision_quantized_act_amd as qa
    from oracle import quant as Q
    t = torch()
    M, H = 777, 1920                      # a ragged element count per vector sweep
    x = synth.activations(4, M, H, "normal")
    d = synth.gamma_pair(4, x, 0.05)
    delta = T.tdc_update(x.ravel(), d.ravel())[0].reshape(M, H)
    xd, dd = dev(x).view(-1), dev(delta).view(-1)
    rws = qa.workspace(qa.reduce_workspace(M * H))
    o0 = t.empty(M * H, dtype=t.int16, device="cuda")
    o1 = t.empty(M * H, dtype=t.int16, device="cuda")
    s0 = t.zeros(2, dtype=t.float64, device="cuda")
    s1 = t.zeros(2, dtype=t.float64, device="cuda")
    qws = qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, H))
    qws.zero_()
    qa.tdc_apply(xd, dd, o0, s0, rws)
    qa.tdc_apply_amax(xd, dd, o1, qws[:4096].view(t.int32), s1, rws)
    t.cuda.synchronize()
    ob = host(o1).view(np.uint16)
    np.testing.assert_array_equal(ob, host(o0).view(np.uint16))
    np.testing.assert_array_equal(host(s1), host(s0))
    want = int((ob.astype(np.uint32) & 0x7FFF).max()) << 16
    assert int(host(qws[:4096].view(t.int32)).astype(np.int64).max()) == want
    c0, sc0, ts0 = qa.empty_nvfp4(M, H)
    c1, sc1, ts1 = qa.empty_nvfp4(M, H)
    qa.act_quant(qa.NVFP4, o0.view(M, H), c0, sc0, ts0, 0,
                 qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, H)))
    qa.act_quant(qa.NVFP4, o1.view(M, H), c1, sc1, ts1, qa.AMAX_GIVEN, qws)
    t.cuda.synchronize()
    for u, v in ((c0, c1), (sc0, sc1), (ts0, ts1)):
        np.testing.assert_array_equal(host(u), host(v))
    oc, osc, ots = Q.nvfp4_encode(ob.reshape(M, H))
    np.testing.assert_array_equal(host(c1), oc)
    assert host(ts1)[0] == ots
