"""Dequantize-then-float64 GEMM of the quantized linear.

Test infrastructure (see the package docstring).

6Bit-Diffusion, abstract and Fig. 2 caption: every internal linear layer of
a DiT block runs with 4-bit weights (Table 2, "W4") and activations in NVFP4
or INT8 chosen per layer.  What the layer computes, written as its plain
definition:  Y = dequant(A) @ dequant(W)^T (+ bias) (-> GELU-tanh), summed
exactly enough in float64 that its error (about K * 2^-53 relative) is far
below any tolerance used against it.  GELU is the tanh form of Hendrycks &
Gimpel, which the pages cite among the works they build on.
"""
import math

import numpy as np

from .formats import bf16_to_f64


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
