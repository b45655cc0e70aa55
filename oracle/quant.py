"""NVFP4 and per-token INT8 quantization of activations and weights.

Test infrastructure (see the package docstring).

6Bit-Diffusion, abstract: each linear layer's activations are quantized at
inference time to NVFP4 (temporally stable layers) or INT8 (volatile
layers); Fig. 2 caption: the DMPQ module chooses the bit width separately
for the activations of every linear layer.  Table 2 runs the weights at 4
bits ("W4").
The pages print no quantizer formula.  The readings taken (all steps in
float32, in this order; recip(y) is 1/y, or 0 when y == 0):

NVFP4 of X[rows, K] (K a multiple of 16), groups of 16 along K:
  1. s_T  = amax(|X|) / 2688            (2688 = 6 * 448: E2M1 max * E4M3 max)
     unless the tensor scale s_T is given by the caller
  2. g    = recip(6 * s_T)
  3. per group: enc = E4M3(amax_group * g)
  4. per group: inv = recip(E4M3value(enc) * s_T)
  5. per element: code = E2M1(x * inv)
  6. codes packed two per byte, element 2j in the low nibble
  Dequantized value: E2M1value(code) * E4M3value(enc) * s_T.

INT8 per token (row) of X[rows, K], symmetric:
  s = amax_row / 127,  inv = recip(s),  q = clamp(rint(x * inv), -127, 127)
  with rint rounding half to even.  Dequantized value: q * s.
"""
import numpy as np

from .formats import (bf16_to_f32, e2m1_decode, e2m1_encode, e4m3_decode,
                      e4m3_encode_nonneg)

F32 = np.float32


def _recip(y):
    y = np.asarray(y, dtype=F32)
    with np.errstate(divide="ignore"):
        r = np.where(y == 0, F32(0), F32(1) / np.where(y == 0, F32(1), y))
    return r.astype(F32)


def nvfp4_tensor_scale(x_bf16):
    """Step 1: s_T = amax / 2688 in float32 (amax of the bf16 tensor)."""
    return _tensor_scale_f32(bf16_to_f32(np.asarray(x_bf16, dtype=np.uint16)))


def _tensor_scale_f32(x):
    amax = F32(np.max(np.abs(x))) if x.size else F32(0)
    return F32(amax / F32(2688.0))


def nvfp4_encode(x_bf16, tscale=None):
    """Quantize bf16 bits X[rows, K] to NVFP4.

    Returns (codes uint8 [rows, K/2], scales uint8 [rows, K/16], s_T float32).
    ``tscale`` given: use it as s_T (step 1 skipped).
    """
    return nvfp4_encode_f32(bf16_to_f32(np.asarray(x_bf16, dtype=np.uint16)), tscale)


def nvfp4_encode_f32(x, tscale=None):
    """The NVFP4 steps on float32 values X[rows, K] (see the module notes)."""
    x = np.asarray(x, dtype=F32)
    rows, K = x.shape
    if K % 16:
        raise ValueError("NVFP4 needs K to be a multiple of 16")
    s_t = _tensor_scale_f32(x) if tscale is None else F32(tscale)
    g = _recip(F32(6.0) * s_t)
    xg = x.reshape(rows, K // 16, 16)
    amax_g = np.max(np.abs(xg), axis=2) if K else np.zeros((rows, 0), F32)
    enc = e4m3_encode_nonneg((amax_g * g).astype(F32))
    d = (e4m3_decode(enc).astype(F32) * s_t).astype(F32)
    inv = _recip(d)
    codes = e2m1_encode((xg * inv[:, :, None]).astype(F32)).reshape(rows, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, enc.astype(np.uint8), F32(s_t)


def nvfp4_unpack(packed):
    """[rows, K/2] bytes -> [rows, K] 4-bit codes (low nibble first)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def nvfp4_decode(packed, scales, tscale):
    """Dequantize NVFP4 to float64: e2m1 * e4m3 * s_T (exact in float64)."""
    codes = nvfp4_unpack(packed)
    rows, K = codes.shape
    v = e2m1_decode(codes).reshape(rows, K // 16, 16)
    s = e4m3_decode(np.asarray(scales, dtype=np.uint8))[:, :, None]
    return (v * s * float(F32(tscale))).reshape(rows, K)


def int8_encode(x_bf16):
    """Per-token symmetric INT8: returns (q int8 [rows, K], s float32 [rows])."""
    return int8_encode_f32(bf16_to_f32(np.asarray(x_bf16, dtype=np.uint16)))


def int8_decode(q, s):
    """q * s in float64 (exact)."""
    return np.asarray(q, dtype=np.float64) * np.asarray(s, dtype=F32).astype(np.float64)[:, None]


def int8_encode_f32(x):
    """The per-token INT8 steps on float32 values X[rows, K]."""
    x = np.asarray(x, dtype=F32)
    rows = x.shape[0]
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(rows, F32)
    s = (amax.astype(F32) / F32(127.0)).astype(F32)
    inv = _recip(s)
    q = np.clip(np.rint((x * inv[:, None]).astype(F32)), -127, 127).astype(np.int8)
    return q, s
