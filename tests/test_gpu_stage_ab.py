"""The compute stages of the three NVFP4 GEMM designs (qa_test_stage_ab:
the library's exact fp16 expansion, design S with fp8 codes and a
per-group rescale, and its fp16 hybrid) against their definitions on one
scale group of 16 K elements, for 16 waves of random operands, decoded
with the oracle's E2M1 and E4M3 tables.  The timing of the same stages is
in bench.py (`design_ab`)."""
import numpy as np
import pytest

from oracle import formats as F
from tests._gpu import host, torch

pytestmark = pytest.mark.gpu

# E4M3 byte of each E2M1 magnitude code (the values 0, .5, 1, 1.5, 2, 3, 4, 6)
E2M1_AS_E4M3 = np.array([0x00, 0x30, 0x38, 0x3C, 0x40, 0x44, 0x48, 0x4C], np.uint32)


def _qa():
    import mixed_precision_quantized_act_amd as qa
    return qa


def _nibbles(words):
    """uint32 [..] -> E2M1 codes [.., 8], element 2i in the low nibble of byte i."""
    w = np.asarray(words, np.uint32)[..., None]
    return ((w >> (4 * np.arange(8, dtype=np.uint32))) & 15).astype(np.uint8)


def _run(design, blk):
    qa, t = _qa(), torch()
    inp = t.from_numpy(blk.view(np.int32).copy()).cuda()
    out = t.full((1024, 256), float("nan"), dtype=t.float32, device="cuda")
    qa._lib.stage_ab(design, 1, 4, inp, out)
    t.cuda.synchronize()
    return host(out)


def _operand(vals):
    """per-lane values [1024, T, 8] (lane's K half) -> per wave and tile the
    32 x 16 operand rows: [16 waves, T, 32 rows, 16 K]."""
    v = vals.reshape(16, 2, 32, vals.shape[1], 8)          # wave, half, row, tile, k
    return np.concatenate([v[:, 0], v[:, 1]], axis=-1).transpose(0, 2, 1, 3)


def _expected(P, scale):
    """P [16 waves, I, J, 32 (W row p), 32 (A row q)] -> per lane, tile (i, j),
    accumulator r the value at p = 8 (r/4) + 4 (l/32) + r % 4, q = l % 32,
    times scale(lane, i, j, r)."""
    waves, I, J = P.shape[:3]
    out = np.zeros((1024, I, J, 16))
    for l in range(64):
        for r in range(16):
            p = 8 * (r // 4) + 4 * (l // 32) + r % 4
            out[np.arange(waves) * 64 + l, :, :, r] = P[:, :, :, p, l % 32]
    return out * scale


@pytest.mark.parametrize("design", [0, 1, 2])
def test_stage_matches_definition(design):
    rng = np.random.default_rng(design)
    blk = np.zeros((1024, 64), np.uint32)
    codes = lambda n: rng.integers(0, 1 << 32, (1024, n), dtype=np.uint64).astype(np.uint32)
    sbytes = lambda n: rng.integers(0x20, 0x60, (1024, n)).astype(np.uint32)   # E4M3 2^-4 .. 2^4
    if design == 0:
        blk[:, 0:4], blk[:, 4:8] = codes(4), codes(4)
        blk[:, 8:12], blk[:, 12:16] = sbytes(4), sbytes(4)
        a = F.e2m1_decode(_nibbles(blk[:, 0:4])) * F.e4m3_decode(blk[:, 8:12])[..., None]
        w = F.e2m1_decode(_nibbles(blk[:, 4:8])) * F.e4m3_decode(blk[:, 12:16])[..., None]
        A, W = _operand(a), _operand(w)                     # [16, 4, 32, 16]
        P = np.einsum("wjpk,wiqk->wijpq", W, A)
        want = _expected(P, 1.0)
        scale = 1.0
        got = _run(0, blk).reshape(1024, 4, 4, 16)
    else:
        sw = F.e4m3_decode(sbytes(48)).astype(np.float32)
        blk[:, 16:64] = sw.view(np.uint32)
        swv = sw.reshape(1024, 3, 16)[:, [0, 1, 2, 0]]       # tile 3 reuses tile 0's
        if design == 1:
            ac, wc = codes(2), codes(4)
            to8 = lambda c: (E2M1_AS_E4M3[_nibbles(c) & 7] | ((_nibbles(c) >> 3) << 7).astype(np.uint32))
            a8, w8 = to8(ac), to8(wc)                        # E4M3 bytes [1024, T, 8]
            pack = lambda b: (b[..., 0::4] | (b[..., 1::4] << 8) | (b[..., 2::4] << 16)
                              | (b[..., 3::4] << 24)).reshape(1024, -1)
            blk[:, 0:4], blk[:, 4:12] = pack(a8), pack(w8)
            sa = F.e4m3_decode(sbytes(2)).astype(np.float32)
            blk[:, 12:14] = sa.view(np.uint32)
            A, W = _operand(F.e2m1_decode(_nibbles(ac))), _operand(F.e2m1_decode(_nibbles(wc)))
            P = np.einsum("wjpk,wiqk->wijpq", W, A)
            scale = sa.astype(np.float64)[:, :, None, None] * swv.astype(np.float64)[:, None, :, :]
        else:
            ac, wc = codes(2), codes(4)
            sab = sbytes(2)
            blk[:, 0:2], blk[:, 2], blk[:, 4:8] = ac, sab[:, 0] | (sab[:, 1] << 8), wc
            a = F.e2m1_decode(_nibbles(ac)) * F.e4m3_decode(sab)[..., None]
            A, W = _operand(a), _operand(F.e2m1_decode(_nibbles(wc)))
            P = np.einsum("wjpk,wiqk->wijpq", W, A)
            scale = swv.astype(np.float64)[:, None, :, :]
        want = _expected(P, scale)
        got = _run(design, blk)[:, :128].reshape(1024, 2, 4, 16)
    # float32 sums of 16 exact products, then at most two roundings of the
    # scaling: within 20 ulp of the sum of the magnitudes
    Pabs = np.einsum("wjpk,wiqk->wijpq", np.abs(W), np.abs(A))
    bound = 20 * 2.0 ** -24 * _expected(Pabs, np.abs(scale) if design else 1.0)
    err = np.abs(got - want)
    assert np.all(err <= bound), float(np.max(err - bound))
