"""Dequantize-then-float64 GEMM of the quantized linear, and the exact
integer accumulators of the INT8-activation path.

Test infrastructure (see the package docstring).

6Bit-Diffusion, abstract and Fig. 2 caption: every internal linear layer of
a DiT block runs with 4-bit weights (Table 2, "W4") and activations in NVFP4
or INT8 chosen per layer.  What the layer computes, written as its plain
definition:  Y = dequant(A) @ dequant(W)^T (+ bias) (-> GELU-tanh), summed
exactly enough in float64 that its error (about K * 2^-53 relative) is far
below any tolerance used against it.  GELU is the tanh form of Hendrycks &
Gimpel, which the pages cite among the works they build on.

The INT8 path's integer accumulators
------------------------------------
An NVFP4 weight element is  s_Tw * (c/2) * M * 2^(F-10)  with c = 2*|E2M1|
in {0,1,2,3,4,6,8,12} (with sign), and the group's E4M3 scale written as an
integer significand M and exponent F:  normal codes (exponent field e >= 1)
give M = 8 + mantissa, F = e;  subnormal codes give M = mantissa, F = 1.
For row n let Fr[n] be the smallest F over the row's groups whose M > 0.
Then  W[n, k] = s_Tw * 2^(Fr[n] - 11) * I[n, k]  with the integer
I = c * M * 2^(F - Fr[n]).  A row is *regular* when its F spread
(max F - Fr over groups with M > 0) is at most 6, so |I| <= 180 * 64.  A
regular row's I splits into two int8 digits, I = 128 * hi + lo with
lo in [-64, 63], and the layer output is
    Y[m, n] = s_a[m] * s_Tw * 2^(Fr[n] - 11) * (128 * ACC_hi + ACC_lo)
with the exact integer sums ACC_x[m, n] = sum_k q[m, k] * x[n, k].
"""
import math

import numpy as np

from .formats import e2m1_decode, bf16_to_f64
from .quant import nvfp4_unpack

SPREAD_MAX = 6


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


def e4m3_sig_exp(scales):
    """Split non-negative E4M3 codes into (M, F) with value M * 2^(F-10)."""
    s = np.asarray(scales, dtype=np.uint8).astype(np.int64)
    e = (s >> 3) & 0xF
    m = s & 7
    sig = np.where(e == 0, m, 8 + m)
    fexp = np.where(e == 0, 1, e)
    return sig, fexp


def weight_integer_repr(w_packed, w_scales):
    """NVFP4 weight -> (I int64 [N,K], Fr int64 [N], regular bool [N]).

    See the module docstring for the definitions.  Rows whose groups all
    have M == 0 are zero; they get Fr = 1 and are regular.
    """
    codes = nvfp4_unpack(w_packed)
    N, K = codes.shape
    c = np.rint(2.0 * e2m1_decode(codes)).astype(np.int64).reshape(N, K // 16, 16)
    sig, fexp = e4m3_sig_exp(w_scales)
    live = sig > 0
    big = np.iinfo(np.int64).max
    fr = np.where(live, fexp, big).min(axis=1) if K else np.full(N, big)
    fr = np.where(fr == big, 1, fr)
    fmax = np.where(live, fexp, 0).max(axis=1) if K else np.zeros(N, np.int64)
    regular = ~live.any(axis=1) | ((fmax - fr) <= SPREAD_MAX)
    shift = np.where(live, fexp - fr[:, None], 0)
    integer = c * (sig * (np.int64(1) << np.maximum(shift, 0)))[:, :, None]
    return integer.reshape(N, K), fr, regular


def int8_digits(integer):
    """I -> (hi, lo) int8 with I = 128*hi + lo, lo in [-64, 63]."""
    integer = np.asarray(integer, dtype=np.int64)
    lo = ((integer + 64) % 128) - 64
    hi = (integer - lo) // 128
    if np.any(np.abs(hi) > 127):
        raise ValueError("row outside the two-digit range")
    return hi.astype(np.int8), lo.astype(np.int8)


def int8_accumulators(q, w_packed, w_scales, rows=None):
    """Exact ACC_hi, ACC_lo (int64 [M, N]) of the regular weight rows.

    Irregular rows are returned as zero columns (their output is formed
    another way and has no such accumulators).  ``rows``: optional subset
    of activation rows.
    """
    integer, _, regular = weight_integer_repr(w_packed, w_scales)
    integer = np.where(regular[:, None], integer, 0)
    hi, lo = int8_digits(integer)
    qa = np.asarray(q, dtype=np.int64)
    if rows is not None:
        qa = qa[rows]
    return qa @ hi.astype(np.int64).T, qa @ lo.astype(np.int64).T
