"""Dequantize-then-float64 GEMM of the quantized linear, and the integer
sums of its INT8-activation path.

Test infrastructure (see the package docstring).

6Bit-Diffusion, abstract and Fig. 2 caption: every internal linear layer of
a DiT block runs with 4-bit weights (Table 2, "W4") and activations in NVFP4
or INT8 chosen per layer.  What the layer computes, written as its plain
definition:  Y = dequant(A) @ dequant(W)^T (+ bias) (-> GELU-tanh), summed
exactly enough in float64 that its error (about K * 2^-53 relative) is far
below any tolerance used against it.  GELU is the tanh form of Hendrycks &
Gimpel, which the pages cite among the works they build on.

The INT8 path's integer sums
----------------------------
With INT8 activations (abstract: volatile layers keep INT8) the linear can
run on integer arithmetic.  An NVFP4 weight element is s_Tw * E4M3 * E2M1.
Write the E4M3 scale as c * 2^x with the integer c of its significand (4
bits for normal codes, the 3 mantissa bits for subnormal ones) and the
E2M1 value as v / 2 with the integer v = 2 * E2M1 in -12..12.  For weight
row n let X[n] be the smallest x over the row's non-zero scales; then
    W[n, k] = s_Tw * 2^(X[n] - 1) * I[n, k],   I = v * c * 2^(x - X[n]),
an integer.  When the row's x values span at most 7 (SPREAD_MAX), |I| is
at most 12 * 15 * 2^7 = 23040 and I has two int8 digits,
    I = 256 * hi + lo,  lo in [-128, 127],  |hi| <= 90,
so that the linear is
    Y[m, n] = s_a[m] * s_Tw * 2^(X[n] - 1) * (256 * H[m, n] + L[m, n])
with the exact integer sums H = sum_k q[m, k] hi[n, k] and
L = sum_k q[m, k] lo[n, k].  Rows with a wider span are "irregular": they
have no two-digit form.
"""
import math

import numpy as np

from .formats import bf16_to_f64, e2m1_decode, e4m3_decode
from .quant import nvfp4_unpack

SPREAD_MAX = 7


def gelu_tanh(x):
    """0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) in float64."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def linear_ref(a_deq, w_deq, bias_bf16=None, gelu=False):
    """Y = A W^T (+ bias) (-> GELU-tanh) in float64; A [M,K], W [N,K]."""
    y = np.asarray(a_deq, dtype=np.float64) @ np.asarray(w_deq, dtype=np.float64).T
    if bias_bf16 is not None:
        y = y + bf16_to_f64(bias_bf16)[None, :]
    if gelu:
        y = gelu_tanh(y)
    return y


def e4m3_significand_exponent(scales):
    """E4M3 scale codes -> (c, x) int64 arrays with value = c * 2^x.

    From the decoded value s: s = f * 2^E with f in [0.5, 1) (frexp), and
    the E4M3 significand has 4 bits (quantum 2^(E-4)) down to the subnormal
    quantum 2^-9, so x = max(E - 4, -9) and c = s / 2^x, an integer 0..15.
    """
    s = e4m3_decode(np.asarray(scales, dtype=np.uint8))
    _, e = np.frexp(s)
    x = np.maximum(e - 4, -9).astype(np.int64)
    c = np.ldexp(s, -x)
    if np.any(c != np.rint(c)):
        raise AssertionError("E4M3 value with more than 4 significant bits")
    return np.rint(c).astype(np.int64), x


def int8_weight_integers(w_packed, w_scales):
    """NVFP4 weight [N, K] -> (I int64 [N, K], X int64 [N], regular bool [N]).

    See the module notes.  Rows without a non-zero scale are zero and
    regular (X = 0); irregular rows (span of x above SPREAD_MAX) get I = 0.
    """
    codes = nvfp4_unpack(w_packed)
    N, K = codes.shape
    v = np.rint(2.0 * e2m1_decode(codes)).astype(np.int64).reshape(N, K // 16, 16)
    c, x = e4m3_significand_exponent(w_scales)
    live = c > 0
    big = np.int64(1 << 20)
    xmin = np.where(live, x, big).min(axis=1) if K else np.full(N, big)
    xmax = np.where(live, x, -big).max(axis=1) if K else np.full(N, -big)
    any_live = live.any(axis=1) if K else np.zeros(N, bool)
    regular = ~any_live | (xmax - xmin <= SPREAD_MAX)
    X = np.where(any_live, xmin, 0)
    shift = np.where(live & regular[:, None], x - X[:, None], 0)
    mult = np.where(live & regular[:, None], c * (np.int64(1) << shift), 0)
    integer = (v * mult[:, :, None]).reshape(N, K)
    return integer, X, regular


def int8_digits(integer):
    """I -> (hi, lo) int8 with I = 256 hi + lo, lo in [-128, 127]."""
    integer = np.asarray(integer, dtype=np.int64)
    lo = (integer + 128) % 256 - 128
    hi = (integer - lo) // 256
    if np.any(np.abs(hi) > 127):
        raise ValueError("value outside the two-digit range")
    return hi.astype(np.int8), lo.astype(np.int8)


def int8_accumulators(q, hi, lo):
    """Exact H = q @ hi^T and L = q @ lo^T (int64 [M, N]).

    Summed in float64, which is exact here: every partial sum is an integer
    below K * 127 * 128 < 2^53.
    """
    qa = np.asarray(q, dtype=np.float64)
    H = qa @ np.asarray(hi, dtype=np.float64).T
    L = qa @ np.asarray(lo, dtype=np.float64).T
    return H.astype(np.int64), L.astype(np.int64)


def int8_linear_from_sums(H, L, X, s_a, w_ts):
    """Y = s_a[m] s_Tw 2^(X[n] - 1) (256 H + L) in float64 (the module notes)."""
    t = 256.0 * np.asarray(H, dtype=np.float64) + np.asarray(L, dtype=np.float64)
    col = np.ldexp(1.0, np.asarray(X, dtype=np.int64) - 1)
    row = np.asarray(s_a, dtype=np.float32).astype(np.float64) * float(np.float32(w_ts))
    return t * col[None, :] * row[:, None]
