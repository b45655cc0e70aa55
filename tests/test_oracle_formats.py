"""Pins of the format encoders in oracle/formats.py.

Each encoder is checked against (a) hand-worked tables in tests/golden,
(b) an independent characterisation: the E2M1 decision thresholds, an
exhaustive argmin over every representable value, the field-by-field
definition of E4M3, and exact rational rounding for bfloat16.
"""
import fractions
import math

import numpy as np
import pytest

from oracle import formats as F
from tests._golden import lines


def test_e2m1_hand_table():
    for v, code, *_ in lines("e2m1_encode.txt"):
        got = F.e2m1_encode(np.float32(float(v)))
        assert int(got) == int(code, 16), (v, code, int(got))


def _e2m1_threshold_rule(a):
    # Ties to the even code put the inclusive side of each decision
    # threshold on the even neighbour: codes 0|1 at .25 (>), 1|2 at .75 (>=),
    # 2|3 at 1.25 (>), 3|4 at 1.75 (>=), 4|5 at 2.5 (>), 5|6 at 3.5 (>=),
    # 6|7 at 5 (>).
    return ((a > 0.25).astype(int) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
            + (a > 2.5) + (a >= 3.5) + (a > 5.0))


def test_e2m1_against_thresholds_random():
    rng = np.random.default_rng(1234)
    v = np.concatenate([rng.standard_normal(2_000_000).astype(np.float32) * 3,
                        rng.uniform(-8, 8, 1_000_000).astype(np.float32),
                        # every tie point and its float32 neighbours
                        np.array([t * s for t in (.25, .75, 1.25, 1.75, 2.5, 3.5, 5.0)
                                  for s in (1, -1)], np.float32)])
    ties = v[-14:]
    v = np.concatenate([v, np.nextafter(ties, np.float32(np.inf)),
                        np.nextafter(ties, np.float32(-np.inf))])
    got = F.e2m1_encode(v)
    want = _e2m1_threshold_rule(np.abs(v).astype(np.float64)) | (np.signbit(v).astype(int) << 3)
    np.testing.assert_array_equal(got, want.astype(np.uint8))


def test_e2m1_against_bruteforce_argmin():
    # nearest of the 8 magnitudes by exhaustive distance, ties to even code
    rng = np.random.default_rng(7)
    a = np.abs(rng.standard_normal(200_000).astype(np.float32) * 2.5)
    a = np.concatenate([a, np.arange(0, 7.5, 0.125, dtype=np.float32)])
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float64)
    dist = np.abs(a[:, None].astype(np.float64) - grid[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among equally near codes take the even one (each tie has one)
    want = np.where(cand.sum(1) == 1, cand.argmax(1),
                    np.argmax(cand & (np.arange(8) % 2 == 0)[None, :], axis=1))
    np.testing.assert_array_equal(F.e2m1_encode(a), want.astype(np.uint8))


def test_e2m1_decode_fields():
    # E2M1 fields: sign | 2-bit exponent (bias 1) | 1-bit mantissa
    for c in range(16):
        s = -1.0 if c & 8 else 1.0
        e, m = (c >> 1) & 3, c & 1
        v = s * (m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1))
        assert F.e2m1_decode(np.uint8(c)) == v


def test_e4m3_hand_table():
    for v, code, *_ in lines("e4m3_encode.txt"):
        got = F.e4m3_encode_nonneg(np.float32(float(v)))
        assert int(got) == int(code, 16), (v, code, int(got))


def test_e4m3_values_from_fields():
    # every finite code, decoded from the bit fields with exact fractions
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        if e == 0:
            want = fractions.Fraction(m, 8) * fractions.Fraction(1, 64)
        else:
            want = (1 + fractions.Fraction(m, 8)) * fractions.Fraction(2) ** (e - 7)
        assert fractions.Fraction(F.E4M3_VAL[c]) == want
        assert F.e4m3_decode(np.uint8(c)) == float(want)
        assert F.e4m3_decode(np.uint8(c | 0x80)) == -float(want)
    assert F.E4M3_MAX == 448.0
    assert math.isnan(F.e4m3_decode(np.uint8(0x7F)))


def test_e4m3_against_bruteforce():
    # exhaustive distance to all 127 values, ties to the even code
    rng = np.random.default_rng(11)
    a = np.concatenate([np.exp(rng.uniform(np.log(1e-4), np.log(600), 100_000)),
                        F.E4M3_VAL, (F.E4M3_VAL[1:] + F.E4M3_VAL[:-1]) / 2]).astype(np.float32)
    vals = F.E4M3_VAL
    dist = np.abs(a[:, None].astype(np.float64) - vals[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    want = np.where(cand.sum(1) == 1, cand.argmax(1),
                    np.argmax(cand & (np.arange(127) % 2 == 0)[None, :], axis=1))
    np.testing.assert_array_equal(F.e4m3_encode_nonneg(a), want.astype(np.uint8))


def test_e4m3_rejects_negative():
    with pytest.raises(ValueError):
        F.e4m3_encode_nonneg(np.float32(-1.0))


def _bf16_exact(x):
    """Nearest bf16 (ties to even) by exact rational arithmetic."""
    fx = fractions.Fraction(x)
    if fx == 0:
        return 0.0
    mag = abs(fx)
    e = math.floor(math.log2(mag))
    while fractions.Fraction(2) ** e > mag:
        e -= 1
    while fractions.Fraction(2) ** (e + 1) <= mag:
        e += 1
    q = fractions.Fraction(2) ** max(e - 7, -133)
    n = mag / q
    r = math.floor(n)
    rem = n - r
    if rem > fractions.Fraction(1, 2) or (rem == fractions.Fraction(1, 2) and r % 2 == 1):
        r += 1
    v = r * q
    return float(v) if fx > 0 else -float(v)


def test_bf16_rne_against_exact_rationals():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-6, 6, 3000),
                        # exact ties: a bf16 value plus half its ulp
                        np.array([1 + 2.0 ** -8, 256 + 1.0, 3 * 2.0 ** -8 + 1, -(1 + 3 * 2.0 ** -8)])])
    got = F.bf16_to_f64(F.f64_to_bf16_rne(x))
    want = np.array([_bf16_exact(float(v)) for v in x])
    np.testing.assert_array_equal(got, want)


def test_bf16_roundtrip_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = np.isfinite(F.bf16_to_f64(bits))
    back = F.f64_to_bf16_rne(F.bf16_to_f64(bits[finite]))
    np.testing.assert_array_equal(back, bits[finite])


def test_bf16_overflow_to_inf():
    mx = (2 - 2.0 ** -7) * 2.0 ** 127
    assert F.bf16_to_f64(F.f64_to_bf16_rne(mx + 2.0 ** 118)) == mx
    assert F.bf16_to_f64(F.f64_to_bf16_rne(mx + 2.0 ** 119)) == np.inf
