"""Pins of oracle/gemm.py: hand-worked tiny linears, exact-rational brute
force with an independent decoding of the codes, and closed forms."""
import fractions
import math

import numpy as np
import pytest

from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q
from tests._golden import table

Fr = fractions.Fraction


def _e2m1_value_fields(c):
    # sign | exponent (2 bits, bias 1) | mantissa (1 bit)
    s = -1 if c & 8 else 1
    e, m = (c >> 1) & 3, c & 1
    return s * (Fr(m, 2) if e == 0 else (1 + Fr(m, 2)) * Fr(2) ** (e - 1))


def _e4m3_value_fields(c):
    e, m = (c >> 3) & 15, c & 7
    return Fr(m, 8) * Fr(1, 64) if e == 0 else (1 + Fr(m, 8)) * Fr(2) ** (e - 7)


def _nvfp4_exact(packed, scales, ts):
    rows, half = packed.shape
    out = [[None] * (2 * half) for _ in range(rows)]
    for r in range(rows):
        for j in range(half):
            b = int(packed[r, j])
            for k, c in ((2 * j, b & 15), (2 * j + 1, b >> 4)):
                out[r][k] = _e2m1_value_fields(c) * _e4m3_value_fields(int(scales[r, k // 16])) * Fr(float(ts))
    return out


def _w5_operands():
    t_i8 = table("int8_row.txt")
    q = np.zeros((1, 16), np.int8)
    q[0, :8] = [int(v) for v in t_i8["q"]]
    s_a = np.array([float(t_i8["scale"][0])], np.float32)
    t = table("nvfp4_group.txt")
    packed = np.array([[int(v, 16) for v in t["packed"][8:]]], np.uint8)
    scales = np.array([[0x38]], np.uint8)
    return q, s_a, packed, scales


def test_w5_int8_times_nvfp4():
    q, s_a, wp, ws = _w5_operands()
    want = float(table("gemm_small.txt")["w5_y"][0])
    y = G.linear_ref(Q.int8_decode(q, s_a), Q.nvfp4_decode(wp, ws, np.float32(1)))
    assert y[0, 0] == want
    # the integer sum of the worked example, from the field decoding
    p = sum(int(q[0, k]) * _e2m1_value_fields(int(c)) * 2
            for k, c in enumerate(Q.nvfp4_unpack(wp)[0]))
    assert p == int(table("gemm_small.txt")["w5_p"][0])
    assert float(s_a[0]) * p / 2 == want


def test_w6_nvfp4_times_nvfp4():
    _, _, wp, ws = _w5_operands()
    d = Q.nvfp4_decode(wp, ws, np.float32(1))
    assert G.linear_ref(d, d)[0, 0] == float(table("gemm_small.txt")["w6_y"][0])


def test_all_ones_codes_give_k():
    K = 64
    packed = np.full((3, K // 2), 0x22, np.uint8)      # e2m1 1.0 in both nibbles
    scales = np.full((3, K // 16), 0x38, np.uint8)     # 1.0
    d = Q.nvfp4_decode(packed, scales, np.float32(1))
    assert np.all(G.linear_ref(d, d) == K)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_rational_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    M, N, K = 5, 4, 48
    ap = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wp = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    as_ = rng.integers(0x28, 0x50, (M, K // 16), dtype=np.uint8)
    ws = rng.integers(0x28, 0x50, (N, K // 16), dtype=np.uint8)
    ta, tw = np.float32(0.25), np.float32(2.0)
    bias = F.f64_to_bf16_rne(rng.standard_normal(N))
    y = G.linear_ref(Q.nvfp4_decode(ap, as_, ta), Q.nvfp4_decode(wp, ws, tw), bias)
    A = _nvfp4_exact(ap, as_, ta)
    W = _nvfp4_exact(wp, ws, tw)
    for m in range(M):
        for n in range(N):
            exact = sum(A[m][k] * W[n][k] for k in range(K)) + Fr(float(F.bf16_to_f64(bias[n])))
            assert y[m, n] == float(exact), (m, n)


def test_exact_rational_general_tensor_scale():
    rng = np.random.default_rng(9)
    x = F.f64_to_bf16_rne(rng.standard_normal((4, 32)) * 3)
    w = F.f64_to_bf16_rne(rng.standard_normal((3, 32)) * 0.02)
    ap, as_, ta = Q.nvfp4_encode(x)
    wp, ws, tw = Q.nvfp4_encode(w)
    y = G.linear_ref(Q.nvfp4_decode(ap, as_, ta), Q.nvfp4_decode(wp, ws, tw))
    A, W = _nvfp4_exact(ap, as_, ta), _nvfp4_exact(wp, ws, tw)
    for m in range(4):
        for n in range(3):
            exact = sum(A[m][k] * W[n][k] for k in range(32))
            assert abs(y[m, n] - float(exact)) <= 4 * 2.0 ** -53 * float(
                sum(abs(A[m][k] * W[n][k]) for k in range(32)))


def test_gelu_tanh_closed_forms():
    assert G.gelu_tanh(0.0) == 0.0
    # large |x|: tanh saturates, GELU -> x (positive) or 0 (negative)
    assert G.gelu_tanh(20.0) == 20.0
    assert abs(G.gelu_tanh(-20.0)) < 1e-300 or G.gelu_tanh(-20.0) == 0.0
    # odd part: gelu(x) - gelu(-x) = x
    x = np.linspace(-5, 5, 101)
    np.testing.assert_allclose(G.gelu_tanh(x) - G.gelu_tanh(-x), x, rtol=0, atol=1e-14)
    # x = 1: 0.5 * (1 + tanh(sqrt(2/pi) * 1.044715))
    assert abs(G.gelu_tanh(1.0) - 0.5 * (1 + math.tanh(math.sqrt(2 / math.pi) * 1.044715))) < 1e-15


# ---------------------------------------------------------------- GELU --

def _gelu_exact(x):
    # x * Phi(x), Phi the standard normal CDF (math.erf)
    return x * 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))


def test_gelu_tanh_close_to_exact_gelu():
    """The tanh form approximates x * Phi(x) uniformly.  Bound: on a grid of
    step h = 1e-3 over [-12, 12] the difference d = gelu_tanh - x Phi(x) stays
    within 4.8e-4 (its largest value, near |x| = 2.7, is 4.73e-4); between
    grid points |d| can grow by at most h/2 * sup|d'| < 1e-5 (|d'| < 0.02);
    outside [-12, 12] both forms agree with max(x, 0) to 1e-30.  So
    |d| <= 5e-4 everywhere.  A dropped cubic term (difference 0.033 at x = 2),
    a wrong coefficient or a missing factor 1/2 breaks the bound."""
    xs = np.arange(-12.0, 12.0 + 1e-9, 1e-3)
    got = G.gelu_tanh(xs)
    want = np.array([_gelu_exact(float(v)) for v in xs])
    assert np.max(np.abs(got - want)) <= 5e-4


def test_gelu_tanh_is_the_tanh_approximation():
    """It is the tanh approximation, not the exact GELU: the two differ by
    more than 1e-4 at x = 1 and x = 2.7, and not at all for large |x|."""
    assert abs(float(G.gelu_tanh(1.0)) - _gelu_exact(1.0)) > 1e-4
    assert abs(float(G.gelu_tanh(-2.7)) - _gelu_exact(-2.7)) > 4e-4
    for x in (-30.0, 30.0):
        assert float(G.gelu_tanh(x)) == pytest.approx(max(x, 0.0), abs=1e-12)


def test_gelu_tanh_odd_part_and_origin():
    """GELU(x) - GELU(-x) = x and GELU(0) = 0, GELU'(0) = 1/2."""
    xs = np.linspace(-6, 6, 241)
    assert np.allclose(G.gelu_tanh(xs) - G.gelu_tanh(-xs), xs, atol=1e-12)
    h = 1e-6
    assert float(G.gelu_tanh(0.0)) == 0.0
    assert (float(G.gelu_tanh(h)) - float(G.gelu_tanh(-h))) / (2 * h) == pytest.approx(0.5, abs=1e-9)


# ------------------------------------------- INT8 path: integer form, digits --

def _pack(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def test_w5_integer_form():
    t = table("gemm_small.txt")
    q, s_a, wp, ws = _w5_operands()
    integer, X, regular = G.int8_weight_integers(wp, ws)
    assert regular.all() and int(X[0]) == int(t["w5_X"][0])
    hi, lo = G.int8_digits(integer)
    H, L = G.int8_accumulators(q, hi, lo)
    assert int(H[0, 0]) == int(t["w5_H"][0]) and int(L[0, 0]) == int(t["w5_L"][0])
    y = G.int8_linear_from_sums(H, L, X, s_a, 1.0)
    assert y[0, 0] == float(t["w5_y"][0])


def test_two_digit_row_by_hand():
    t = table("gemm_small.txt")
    codes = np.zeros((1, 32), np.uint8)
    codes[0, 0], codes[0, 16], codes[0, 17] = 0x1, 0x7, 0xB
    scales = np.array([[0x40, 0x7E]], np.uint8)
    integer, X, regular = G.int8_weight_integers(_pack(codes), scales)
    assert regular[0] and int(X[0]) == int(t["d2_X"][0])
    hi, lo = G.int8_digits(integer)
    assert (int(hi[0, 16]), int(lo[0, 16])) == (int(t["d2_hi16"][0]), 0)
    assert (int(hi[0, 17]), int(lo[0, 17])) == (int(t["d2_hi17"][0]), 0)
    assert (int(hi[0, 0]), int(lo[0, 0])) == (0, 8)
    q = np.zeros((1, 32), np.int8)
    q[0, 0], q[0, 16], q[0, 17] = 3, 2, -1
    H, L = G.int8_accumulators(q, hi, lo)
    assert (int(H[0, 0]), int(L[0, 0])) == (int(t["d2_H"][0]), int(t["d2_L"][0]))
    y = G.int8_linear_from_sums(H, L, X, np.ones(1, np.float32), 1.0)
    assert y[0, 0] == float(t["d2_y"][0])
    # the same through the dequantized float64 reference
    ref = G.linear_ref(q.astype(np.float64), Q.nvfp4_decode(_pack(codes), scales, np.float32(1)))
    assert ref[0, 0] == float(t["d2_y"][0])


def test_span_eight_is_irregular():
    codes = np.zeros((2, 32), np.uint8)
    codes[:, 0] = 0x7
    scales = np.array([[0x38, 0x7E], [0x40, 0x7E]], np.uint8)   # spans 8 and 7
    integer, _, regular = G.int8_weight_integers(_pack(codes), scales)
    assert list(regular) == [False, True]
    assert not integer[0].any()


def test_significand_exponent_of_every_e4m3_code():
    """c * 2^x equals the field-decoded value of each of the 127 finite
    non-negative codes, with c a 4-bit integer (8..15 for normal codes)."""
    codes = np.arange(0x7F, dtype=np.uint8)
    c, x = G.e4m3_significand_exponent(codes)
    for code in range(0x7F):
        assert Fr(int(c[code])) * Fr(2) ** int(x[code]) == _e4m3_value_fields(code)
        assert 0 <= c[code] <= 15
        if code >> 3:
            assert 8 <= c[code] <= 15
    assert (int(c[0x38]), int(x[0x38])) == (8, -3) and (int(c[0x7E]), int(x[0x7E])) == (14, 5)


def _random_weight(rng, N, K, span):
    """NVFP4 weight rows with group-scale exponents drawn over `span` octaves
    (subnormal scales included for span >= 9)."""
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    lo_code = max(0x01, 0x7E - 8 * (span + 1))
    scales = rng.integers(lo_code, 0x7F, size=(N, K // 16), dtype=np.uint8)
    zero = rng.random((N, K // 16)) < 0.1
    scales = np.where(zero, 0, scales).astype(np.uint8)
    return _pack(codes), scales


@pytest.mark.parametrize("span", [0, 3, 7, 9, 14])
def test_integer_form_is_exact(span):
    """Brute force: for every element of regular rows, 2^(X-1) * I equals the
    field-decoded E2M1 x E4M3 value exactly; the digits recombine to I and
    stay in range; irregular rows are exactly those whose non-zero scales
    span more than 7 octaves (checked from the field decoding)."""
    rng = np.random.default_rng(100 + span)
    N, K = 24, 64
    wp, ws = _random_weight(rng, N, K, span)
    integer, X, regular = G.int8_weight_integers(wp, ws)
    hi, lo = G.int8_digits(integer)
    assert np.array_equal(256 * hi.astype(np.int64) + lo, integer)
    assert lo.min() >= -128 and lo.max() <= 127 and np.abs(hi.astype(np.int64)).max() <= 90
    codes = Q.nvfp4_unpack(wp)
    for n in range(N):
        ex = []
        for gi in range(K // 16):
            v = _e4m3_value_fields(int(ws[n, gi]))
            if v:
                ex.append(math.frexp(float(v))[1])
        # octave span of the non-zero scales (subnormals share the lowest octave)
        oct_ = [max(e - 4, -9) for e in ex]
        want_regular = not oct_ or max(oct_) - min(oct_) <= 7
        assert bool(regular[n]) == want_regular
        if not want_regular:
            continue
        for k in range(K):
            exact = _e2m1_value_fields(int(codes[n, k])) * _e4m3_value_fields(int(ws[n, k // 16]))
            assert Fr(int(integer[n, k])) * Fr(2) ** (int(X[n]) - 1) == exact


def test_accumulators_brute_force():
    """H and L against explicit integer double loops, and the recombined
    output against the exact rational sum of the dequantized products."""
    rng = np.random.default_rng(7)
    M, N, K = 5, 6, 48
    wp, ws = _random_weight(rng, N, K, 5)
    q = rng.integers(-127, 128, size=(M, K), dtype=np.int64).astype(np.int8)
    s_a = rng.uniform(0.01, 2.0, M).astype(np.float32)
    w_ts = np.float32(0.37)
    integer, X, regular = G.int8_weight_integers(wp, ws)
    assert regular.all()
    hi, lo = G.int8_digits(integer)
    H, L = G.int8_accumulators(q, hi, lo)
    exact_w = _nvfp4_exact(wp, ws, w_ts)
    y = G.int8_linear_from_sums(H, L, X, s_a, w_ts)
    for m in range(M):
        for n in range(N):
            assert H[m, n] == sum(int(q[m, k]) * int(hi[n, k]) for k in range(K))
            assert L[m, n] == sum(int(q[m, k]) * int(lo[n, k]) for k in range(K))
            exact = sum(Fr(int(q[m, k])) * Fr(float(s_a[m])) * exact_w[n][k] for k in range(K))
            assert abs(Fr(float(y[m, n])) - exact) <= abs(exact) * Fr(1, 2 ** 50)
