"""Pins of oracle/tdc.py: hand-worked Gamma, predictor and TDC cases,
closed forms, and the skip pattern of the state machine on scripted runs."""
import copy
import fractions
from fractions import Fraction
import math

import numpy as np

from oracle import formats as F
from oracle import tdc as T
from tests._golden import table

Fr = fractions.Fraction


def _bf16(v):
    return F.f64_to_bf16_rne(np.asarray(v, dtype=np.float64))


def _row(t, key):
    return [float(v) for v in t[key]]


def test_w7_gamma_and_rule():
    t = table("gamma_dmpq.txt")
    x, y = _bf16(_row(t, "in")), _bf16(_row(t, "out"))
    g = T.gamma(x, y)
    assert g == float(t["gamma"][0])
    alpha, beta = np.float32(1.0), np.float32(2.0 ** -7)
    p = T.predictions([g], [alpha], [beta], 1)[0]
    assert p == float(t["p"][0])
    assert T.dmpq_mask([g], [alpha], [beta], p, 1)[0] == int(t["mask_at_tau_eq_p"][0])
    assert T.dmpq_mask([g], [alpha], [beta], 0.125, 1)[0] == int(t["mask_at_tau_0.125"][0])


def test_gamma_closed_forms():
    rng = np.random.default_rng(1)
    x = _bf16(rng.standard_normal(1000))
    xf = F.bf16_to_f64(x)
    assert T.gamma(x, x) == 0.0
    assert T.gamma(x, _bf16(2 * xf)) == 1.0
    assert T.gamma(x, _bf16(-xf)) == 2.0
    z = np.zeros(4, np.uint16)
    assert T.gamma(z, z) == 0.0
    assert T.gamma(z, _bf16([1, 0, 0, 0])) == math.inf


def test_gamma_sums_exact():
    rng = np.random.default_rng(2)
    x = _bf16(rng.standard_normal(500))
    y = _bf16(F.bf16_to_f64(x) + 0.1 * rng.standard_normal(500))
    s1, s2 = T.gamma_sums(x, y)
    e1 = sum(abs(Fr(float(b)) - Fr(float(a))) for a, b in zip(F.bf16_to_f64(x), F.bf16_to_f64(y)))
    e2 = sum(abs(Fr(float(a))) for a in F.bf16_to_f64(x))
    assert s1 == float(e1) and s2 == float(e2)


def test_dmpq_first_step_all_int8_and_layout():
    a = np.array([1, 1, 2, 2], np.float32)
    b = np.array([0, 0.5, 0, 0], np.float32)
    assert T.dmpq_mask(None, a, b, 0.3, 2).tolist() == [1, 1, 1, 1]
    # gamma per block repeats over its J linears: block 0 -> 0.1, block 1 -> 0.2
    assert T.dmpq_mask([0.1, 0.2], a, b, 0.3, 2).tolist() == [0, 1, 1, 1]


def test_tau_for_half():
    assert T.tau_for_half([4, 1, 3, 2]) == 2.5
    p = np.random.default_rng(3).standard_normal(40)
    assert (p > T.tau_for_half(p)).sum() == 20


def test_w8_relative_l2_and_decision():
    t = table("tdc.txt")
    older = _bf16(_row(t, "delta_older"))
    for key, dkey, skip in (("delta_newer_a", "d_a", 1), ("delta_newer_b", "d_b", 0)):
        newer = _bf16(_row(t, key))
        # in = 0 makes out - in = Delta exactly
        zero = np.zeros_like(newer)
        dn, sums = T.tdc_update(zero, newer, older)
        np.testing.assert_array_equal(dn, newer)
        d = T.rel_l2(sums[2], sums[3])
        assert d == float(t[dkey][0])
        assert T.tdc_decide(2, [d], [True], 0.05)[0] == skip


def test_w8_rounding():
    t = table("tdc.txt")
    out = T.tdc_apply(_bf16(_row(t, "apply_in")), _bf16(_row(t, "apply_delta")))
    assert F.bf16_to_f64(out).tolist() == _row(t, "apply_out")
    d, _ = T.tdc_update(_bf16(_row(t, "delta_in")), _bf16(_row(t, "delta_out")))
    assert F.bf16_to_f64(d).tolist() == _row(t, "delta")


def test_decide_rules():
    assert T.tdc_decide(1, [0.0], [True], 0.05).tolist() == [0]   # warm-up
    assert T.tdc_decide(2, [0.0], [False], 0.05).tolist() == [0]  # skipped at t-1
    assert T.tdc_decide(2, [0.05], [True], 0.05).tolist() == [0]  # equality computes
    assert T.tdc_decide(2, [0.0499], [True], 0.05).tolist() == [1]


def _run_block(deltas, steps=10, delta=0.05, start=None, t0=0):
    """Drive one block: x_t drifts, a computed block outputs x + deltas(t)."""
    rng = np.random.default_rng(77)
    cache = start if start is not None else T.BlockCache()
    pattern, outs = [], []
    x = rng.standard_normal(64)
    for t in range(steps):
        x = x + 0.02 * rng.standard_normal(64)
        if t < t0:
            continue
        xin = _bf16(x)
        skip = T.tdc_decide(t, [cache.d_prev], [cache.computed_prev], delta)[0]
        if skip:
            out = cache.skip_output(xin)
            pattern.append("S")
        else:
            out = _bf16(F.bf16_to_f64(xin) + deltas(t))
            cache.computed(xin, out)
            pattern.append("C")
        outs.append(out)
    return pattern, outs, cache


def test_state_machine_patterns():
    t = table("tdc.txt")
    base = np.linspace(-1, 1, 64)
    const, _, _ = _run_block(lambda s: base)
    # a constant target output residual still wobbles by bf16 rounding of
    # out relative to a drifting in, which stays far below delta
    assert const == t["pattern_constant"]
    grow, _, _ = _run_block(lambda s: base * 1.0625 ** s)
    assert grow == t["pattern_growing"]


def test_checkpoint_restore_identical():
    base = np.linspace(-1, 1, 64)
    full_pat, full_out, _ = _run_block(lambda s: base)
    # run 0..4, snapshot the cache, continue 5..9 from the snapshot
    _, _, mid = _run_block(lambda s: base, steps=5)
    snap = copy.deepcopy(mid)
    pat2, out2, _ = _run_block(lambda s: base, steps=10, start=snap, t0=5)
    assert full_pat[5:] == pat2
    for a, b in zip(full_out[5:], out2):
        np.testing.assert_array_equal(a, b)


def test_fp32_then_bf16_equals_exact_rounding():
    # Delta = bf16(out - in) and out = bf16(in + Delta) round the exact value
    # once; forming the sum in float32 first gives the same bf16 (float32
    # keeps 24 >= 2*8 + 2 bits, so the second rounding is innocuous)
    rng = np.random.default_rng(4)
    a = _bf16(rng.standard_normal(200_000) * 10.0 ** rng.integers(-3, 4, 200_000))
    b = _bf16(rng.standard_normal(200_000) * 10.0 ** rng.integers(-3, 4, 200_000))
    fa, fb = F.bf16_to_f32(a), F.bf16_to_f32(b)
    via32 = F.f32_to_bf16_rne((fb - fa).astype(np.float32))
    exact = T.tdc_update(a, b)[0]
    np.testing.assert_array_equal(via32, exact)
    np.testing.assert_array_equal(F.f32_to_bf16_rne((fa + fb).astype(np.float32)), T.tdc_apply(a, b))


def test_pairwise_sums_within_bound():
    rng = np.random.default_rng(9)
    x = _bf16(rng.standard_normal(1 << 20))
    y = _bf16(F.bf16_to_f64(x) + 0.05 * rng.standard_normal(1 << 20))
    p = rng.standard_normal(1 << 20)
    pb = _bf16(p)
    _, exact = T.tdc_update(x, y, pb)
    _, pair = T.tdc_update(x, y, pb, summation="pairwise")
    for a, b in zip(exact, pair):
        assert abs(a - b) <= 21 * 2.0 ** -53 * abs(a)


# ---- E_rel and the predictor fit (Fig. 3 caption) ----

def test_rel_err_worked_values():
    # reference (3, 4) has norm 5; output (3, 5) differs by (0, 1): E_rel = 1/5
    ref = F.f64_to_bf16_rne(np.array([3.0, 4.0]))
    out = F.f64_to_bf16_rne(np.array([3.0, 5.0]))
    s0, s1 = T.rel_err_sums(out, ref)
    assert (s0, s1) == (1.0, 25.0)
    assert T.rel_err(s0, s1) == 0.2
    z = F.f64_to_bf16_rne(np.zeros(2))
    assert T.rel_err(*T.rel_err_sums(z, z)) == 0.0
    assert T.rel_err(*T.rel_err_sums(out, z)) == math.inf


def test_rel_err_equals_norm_ratio():
    rng = np.random.default_rng(7)
    r = F.f64_to_bf16_rne(rng.standard_normal(999))
    q = F.f64_to_bf16_rne(F.bf16_to_f64(r) + 0.01 * rng.standard_normal(999))
    qa, ra = F.bf16_to_f64(q), F.bf16_to_f64(r)
    want = np.linalg.norm(qa - ra) / np.linalg.norm(ra)
    assert abs(T.rel_err(*T.rel_err_sums(q, r)) - want) <= 1e-14 * want


def test_fraction_to_f32_rounding():
    # exact float32 values stay; halfway cases go to even; matches numpy's
    # correctly rounded float64 -> float32 where the input is a float64
    assert T.fraction_to_f32(Fraction(3, 4)) == np.float32(0.75)
    one_ulp = Fraction(1, 2 ** 23)
    assert T.fraction_to_f32(1 + one_ulp / 2) == np.float32(1.0)            # tie -> even
    assert T.fraction_to_f32(1 + 3 * one_ulp / 2) == np.float32(1 + 2 * 2 ** -23)
    assert T.fraction_to_f32(-(1 + one_ulp / 2 + Fraction(1, 2 ** 60))) == np.float32(-(1 + 2 ** -23))
    rng = np.random.default_rng(3)
    for v in rng.standard_normal(200) * 10.0 ** rng.integers(-6, 6, 200):
        assert T.fraction_to_f32(Fraction(float(v))) == np.float32(v)


def test_fit_exact_line():
    x = np.array([0.0, 0.125, 0.5, 1.0, 3.0])
    y = 2.5 * x - 0.75                         # exact in binary
    assert T.fit_line(x, y) == (np.float32(2.5), np.float32(-0.75))


def test_fit_matches_polyfit():
    rng = np.random.default_rng(11)
    for _ in range(20):
        n = int(rng.integers(3, 40))
        x = rng.uniform(0, 0.3, n)
        y = 0.8 * x + 0.02 + 0.01 * rng.standard_normal(n)
        a, b = T.fit_line(x, y)
        pa, pb = np.polyfit(x, y, 1)
        assert abs(float(a) - pa) <= 2e-7 * abs(pa) + 1e-12
        assert abs(float(b) - pb) <= 2e-7 * abs(pb) + 1e-12


def test_fit_invariances_and_degenerate():
    rng = np.random.default_rng(12)
    x, y = rng.uniform(0, 1, 9), rng.uniform(0, 1, 9)
    a, b = T.fit_line(x, y)
    a2, b2 = T.fit_line(x, 2 * y)              # scaling by 2 is exact
    assert (a2, b2) == (np.float32(2 * float(a)), np.float32(2 * float(b)))
    a3, b3 = T.fit_line(x, y + 0.5)            # shift moves only beta
    assert a3 == a and abs(float(b3) - (float(b) + 0.5)) <= 2 ** -23
    assert T.fit_line([], []) == (np.float32(0), np.float32(0))
    assert T.fit_line([0.3], [0.7]) == (np.float32(0), np.float32(0.7))
    assert T.fit_line([0.3, 0.3, 0.3], [1.0, 2.0, 6.0]) == (np.float32(0), np.float32(3.0))


def test_calibrate_time_shift():
    # E_rel at t is exactly 3 Gamma_{t-1} + 0.25 for every linear; pairing
    # Gamma_t with E_rel_t instead would not fit a line at all
    rng = np.random.default_rng(13)
    Tn, L, J = 7, 3, 2
    g = rng.uniform(0.01, 0.2, (Tn, L))
    e = np.full((Tn, L * J), np.nan)
    for t in range(1, Tn):
        for l in range(L):
            for j in range(J):
                e[t, l * J + j] = (3.0 + j) * g[t - 1, l] + 0.25
    a, b = T.calibrate(g, e, J)
    for l in range(L):
        for j in range(J):
            assert abs(float(a[l * J + j]) - (3.0 + j)) <= 4e-7 * (3.0 + j)
            assert abs(float(b[l * J + j]) - 0.25) <= 1e-6
    # a non-finite value drops its pair only
    e2 = e.copy()
    e2[3, 0] = np.inf
    a2, _ = T.calibrate(g, e2, J)
    assert abs(float(a2[0]) - 3.0) <= 4e-7 * 3


# ---- cosine similarity of successive Deltas (Fig. 4 caption) ----

def test_cosine_worked_values():
    e1 = F.f64_to_bf16_rne(np.array([1.0, 0.0, 0.0, 0.0]))
    e2 = F.f64_to_bf16_rne(np.array([0.0, 2.0, 0.0, 0.0]))
    v = F.f64_to_bf16_rne(np.array([3.0, 4.0, 0.0, 0.0]))
    assert T.cosine(*T.cosine_sums(e1, e2)) == 0.0                     # orthogonal
    assert T.cosine(*T.cosine_sums(v, v)) == 1.0                       # identical
    neg = F.f64_to_bf16_rne(-F.bf16_to_f64(v))
    assert T.cosine(*T.cosine_sums(v, neg)) == -1.0                    # opposite
    assert T.cosine(*T.cosine_sums(e1, v)) == 0.6                      # 3/5
    z = F.f64_to_bf16_rne(np.zeros(4))
    assert T.cosine(*T.cosine_sums(v, z)) == 0.0                       # zero norm


def test_cosine_matches_numpy_and_scale_invariance():
    rng = np.random.default_rng(5)
    a = F.f64_to_bf16_rne(rng.standard_normal(777))
    b = F.f64_to_bf16_rne(F.bf16_to_f64(a) + 0.3 * rng.standard_normal(777))
    af, bf = F.bf16_to_f64(a), F.bf16_to_f64(b)
    want = float(af @ bf / (np.linalg.norm(af) * np.linalg.norm(bf)))
    got = T.cosine(*T.cosine_sums(a, b))
    assert abs(got - want) <= 1e-14
    b4 = F.f64_to_bf16_rne(4.0 * bf)                                   # exact scaling
    assert abs(T.cosine(*T.cosine_sums(a, b4)) - got) <= 1e-15


def test_decide_cos_rule():
    assert list(T.tdc_decide_cos(1, [0.99, 0.99], [1, 1], 0.9)) == [0, 0]   # warm-up
    assert list(T.tdc_decide_cos(2, [0.99, 0.9, 0.5], [1, 1, 1], 0.9)) == [1, 0, 0]  # strict
    assert list(T.tdc_decide_cos(5, [0.99, 0.99], [0, 1], 0.9)) == [0, 1]   # after a skip
