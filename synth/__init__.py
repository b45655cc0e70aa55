"""Seeded synthetic inputs for the quantized-linear workloads.

This module only draws random numbers and rounds them to bfloat16 once; it
holds none of the quantized linear's arithmetic.  Tests, the smoke check
and the bench draw their inputs here, so the HIP library and the CPU
oracle see the same bytes.

Shapes follow CogVideoX as cited by 6Bit-Diffusion (Table 1 and Table 2 use
CogVideoX-2B; CogVideoX-5B is the larger variant): 17776 tokens (17550
video + 226 text), hidden 1920 (2B) or 3072 (5B), FFN width 4x hidden.  The
pages evaluate on VBench prompts with trained weights; neither is used
here: these seeded Gaussian / Student-t draws stand in for them.

Random streams: ``np.random.default_rng([config_id, stream])`` with stream
0 = activations, 1 = outlier columns, 2 + l = weights of layer l,
50 = the Gamma pair's noise, 100 + t = the drift noise of step t.
"""
import numpy as np

TOKENS = 17776          # 17550 video + 226 text tokens

CONFIGS = {
    1: dict(name="linear-256", M=256, K=256, N=256, dist="normal",
            outliers=4, outlier_mult=20.0),
    2: dict(name="cogvideox2b-qkv", M=TOKENS, K=1920, N=5760, dist="normal",
            outliers=19, outlier_mult=30.0),          # 1 % of 1920 columns
    3: dict(name="cogvideox2b-ffn", M=TOKENS, K=1920, F=7680, dist="t3"),
    4: dict(name="cogvideox2b-stack", M=TOKENS, H=1920, heads=30, F=7680,
            L=30, steps=10, drift=0.02),
    5: dict(name="cogvideox5b-stack", M=TOKENS, H=3072, heads=48, F=12288,
            L=42, steps=10, drift=0.02),
}

WEIGHT_STD = 0.02


def rng(config_id, stream):
    return np.random.default_rng([int(config_id), int(stream)])


def bf16_bits(x):
    """float64 -> bfloat16 bit patterns, one round-to-nearest-even.

    Done on the float64 encoding: keep 7 of the 52 stored mantissa bits,
    adding half of the dropped part (plus the kept LSB for ties) first.
    Valid for finite values inside the bfloat16 normal range, which is all
    these generators produce (and zero).
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_x, flat_o = x.reshape(-1), out.reshape(-1)
    step = 1 << 22
    for i in range(0, flat_x.size, step):
        b = flat_x[i:i + step].view(np.uint64)
        lsb = (b >> np.uint64(45)) & np.uint64(1)
        r = (b + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
        flat_o[i:i + step] = (r.view(np.float64).astype(np.float32).view(np.uint32)
                              >> np.uint32(16)).astype(np.uint16)
    return out


def activations(config_id, M, K, dist="normal", outliers=0, outlier_mult=1.0):
    """[M, K] bf16 activations: N(0,1) or Student-t(3), with ``outliers``
    columns (drawn without replacement) multiplied by ``outlier_mult``."""
    g = rng(config_id, 0)
    if dist == "normal":
        x = g.standard_normal((M, K))
    elif dist == "t3":
        x = g.standard_t(3.0, (M, K))
    else:
        raise ValueError(dist)
    if outliers:
        cols = rng(config_id, 1).choice(K, outliers, replace=False)
        x[:, cols] *= outlier_mult
    return bf16_bits(x)


def weight(config_id, layer, N, K, std=WEIGHT_STD):
    """[N, K] bf16 weight of layer ``layer`` ~ N(0, std^2)."""
    return bf16_bits(rng(config_id, 2 + layer).standard_normal((N, K)) * std)


def gamma_pair(config_id, x_bits, scale=0.1):
    """out = bf16(in + scale * N(0,1)) for a synthetic block in/out pair."""
    x = (np.asarray(x_bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    noise = rng(config_id, 50).standard_normal(x.shape)
    return bf16_bits(x.astype(np.float64) + scale * noise)


def drift(config_id, t, x_bits, scale=0.02):
    """x_t = bf16(x_{t-1} + scale * N(0,1)) with the noise of step t."""
    x = (np.asarray(x_bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    noise = rng(config_id, 100 + t).standard_normal(x.shape)
    return bf16_bits(x.astype(np.float64) + scale * noise)


def linear_case(config_id):
    """(x [M,K], w [N,K]) bf16 bits of a single-linear config (1 or 2)."""
    c = CONFIGS[config_id]
    x = activations(config_id, c["M"], c["K"], c["dist"], c["outliers"], c["outlier_mult"])
    w = weight(config_id, 0, c["N"], c["K"])
    return x, w


def ffn_case(config_id=3, M=None):
    """(x [M,1920], w_up [7680,1920], w_down [1920,7680]) of the FFN config."""
    c = CONFIGS[config_id]
    M = c["M"] if M is None else M
    x = activations(config_id, M, c["K"], c["dist"])
    return x, weight(config_id, 0, c["F"], c["K"]), weight(config_id, 1, c["K"], c["F"])
