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
