"""The C ABI on the host: the library loads, exports every declared entry
point, rejects bad arguments before any launch, and its host-side
decisions equal the oracle's."""
import ctypes
import os
import re

import numpy as np
import pytest

import mixed_precision_quantized_act_amd as qa
from oracle import tdc as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "qact.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\(", src, flags=re.M))


def test_every_declared_symbol_exported_and_bound():
    declared = _declared()
    assert {"act_quant", "qlinear_nvfp4", "qlinear_int8", "block_gamma", "tdc_update",
            "tdc_apply", "dmpq_mask", "tdc_decide"} <= declared
    lib = qa.lib()
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(qa.EXPORTS)


def test_build_info():
    assert "gfx950" in qa.build_info()


FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: every call below fails validation
FAKE_ODD = ctypes.c_void_p(0x10008)


def _status(fn, *args):
    return getattr(qa.lib(), fn)(*args)


def test_act_quant_validation():
    assert _status("act_quant", 0, None, 4, 16, 16, FAKE, FAKE, FAKE, 0, FAKE, 1 << 20, None) == -1
    assert _status("act_quant", 0, FAKE, 4, 24, 24, FAKE, FAKE, FAKE, 0, FAKE, 1 << 20, None) == -2
    assert _status("act_quant", 0, FAKE, 4, 16, 8, FAKE, FAKE, FAKE, 0, FAKE, 1 << 20, None) == -2
    assert _status("act_quant", 0, FAKE_ODD, 4, 16, 16, FAKE, FAKE, FAKE, 0, FAKE, 1 << 20, None) == -3
    assert _status("act_quant", 0, FAKE, 4, 16, 16, FAKE, FAKE, FAKE, 0, FAKE, 0, None) == -5
    assert _status("act_quant", 7, FAKE, 4, 16, 16, FAKE, FAKE, FAKE, 0, FAKE, 1 << 20, None) == -1
    assert _status("act_quant", 1, FAKE, 4, 16, 16, FAKE, FAKE, FAKE, 0, None, 0, None) == -1
    assert _status("act_quant", 0, FAKE, -1, 16, 16, FAKE, FAKE, FAKE, 0, FAKE, 1 << 20, None) == -2
    # unknown flags, and both given-flags at once
    assert _status("act_quant", 0, FAKE, 4, 16, 16, FAKE, FAKE, FAKE, 4, FAKE, 1 << 20, None) == -1
    assert _status("act_quant", 0, FAKE, 4, 16, 16, FAKE, FAKE, FAKE, 3, FAKE, 1 << 20, None) == -1
    # QA_AMAX_GIVEN reads amax from a 4-byte aligned workspace
    assert _status("act_quant", 0, FAKE, 4, 16, 16, ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000),
                   ctypes.c_void_p(0x40000), 2, ctypes.c_void_p(0x50002), 1 << 20, None) == -3
    # q overlapping x
    assert _status("act_quant", 1, FAKE, 4, 16, 16, FAKE, ctypes.c_void_p(0x20000), None, 0,
                   None, 0, None) == -7


def test_qlinear_validation():
    big = 1 << 40
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]
    assert _status("qlinear_nvfp4", *ok, 4, 4, 24, None, ctypes.c_void_p(0x900000), 4, 0, 0, FAKE, big, None) == -2
    assert _status("qlinear_nvfp4", *ok, 4, 4, 16, None, ctypes.c_void_p(0x900000), 3, 0, 0, FAKE, big, None) == -2
    assert _status("qlinear_nvfp4", *ok, 4, 4, 16, None, ctypes.c_void_p(0x900000), 4, 5, 0, FAKE, big, None) == -1
    assert _status("qlinear_nvfp4", *ok, 4, 4, 16, None, ctypes.c_void_p(0x900000), 4, 0, 9, FAKE, big, None) == -1
    assert _status("qlinear_nvfp4", *ok, 4, 4, 16, None, ctypes.c_void_p(0x900000), 4, 0, 0, FAKE, 0, None) == -5
    assert _status("qlinear_nvfp4", None, *ok[1:], 4, 4, 16, None, ctypes.c_void_p(0x900000), 4, 0, 0, FAKE, big, None) == -1
    assert _status("qlinear_int8", *ok[:5], None, 4, 4, 16, None, ctypes.c_void_p(0x900000), 4, 0, 0, FAKE, 0, None) == -5
    assert _status("qlinear_int8", *ok[:5], None, 4, 4, 16, None, ctypes.c_void_p(0x900001), 4, 0, 0, FAKE, big, None) == -3
    # INT8 with K a multiple of 64 reads the weight scales in place, only
    # from a 4-byte aligned array; otherwise the workspace is needed (NVFP4
    # always needs it)
    odd = ctypes.c_void_p(FAKE.value + 1)
    assert _status("qlinear_nvfp4", *ok, 4, 4, 64, None, ctypes.c_void_p(0x900000), 4, 0, 0, None, 0, None) == -5
    assert _status("qlinear_int8", *ok[:3], odd, FAKE, None, 4, 4, 64, None, ctypes.c_void_p(0x900000), 4, 0, 0, None, 0, None) == -5
    assert _status("qlinear_int8", *ok[:5], None, 4, 4, 80, None, ctypes.c_void_p(0x900000), 4, 0, 0, None, 0, None) == -5
    # per-tile copies of the E4M3 scales: 4 bytes per row and K unit of 64,
    # rows rounded up to tiles of 256
    units = (1920 + 63) // 64
    tiles = lambda r: (r + 255) // 256
    r256 = lambda b: (b + 255) // 256 * 256
    # K split of the last round of tiles: 70 x 23 = 1610 tiles are 6 rounds
    # of 256 and 74 more; 3 slices of 10 units would take only 20 units off
    # the last round (less than the 24 a split must save), so no split
    assert qa.qlinear_workspace(qa.NVFP4, 17776, 5760, 1920) == \
        r256(tiles(17776) * units * 1024) + r256(tiles(5760) * units * 1024)
    assert qa.qlinear_workspace(qa.INT8, 17776, 5760, 1920) == r256(tiles(5760) * units * 1024)
    # the down projection: 70 x 8 = 560 = 2 x 256 + 48 tiles, K = 7680 (120
    # units) in 4 slices of 30 (256 // 48 = 5, at most 4): 90 units saved;
    # 256 x 256 fp32 partial sums per slice
    k4 = (7680 + 63) // 64
    assert qa.qlinear_workspace(qa.INT8, 17776, 1920, 7680) == \
        r256(8 * k4 * 1024) + 48 * 4 * 256 * 256 * 4
    # a full last round (8 x 32 = 256 tiles) or one more than half full
    # (13 x 30 = 390 = 256 + 134) is not split
    assert qa.qlinear_workspace(qa.INT8, 2048, 8192, 7680) == r256(32 * k4 * 1024)
    # (with the weight's digit planes the INT8 linear runs 256 x 128 tiles:
    # 13 x 60 = 780 = 3 x 256 + 12, split in 4 slices of int32 partial sums;
    # the workspace covers both INT8 kernels)
    assert qa.qlinear_workspace(qa.INT8, 3328, 7680, 7680) == \
        max(r256(30 * k4 * 1024), 12 * 4 * 256 * 256 * 4)


def test_tdc_validation():
    assert _status("tdc_update", FAKE, FAKE, None, FAKE, 64, FAKE, FAKE, 1 << 20, None) == -7
    assert _status("tdc_update", FAKE, FAKE, None, FAKE_ODD, 64, FAKE, FAKE, 1 << 20, None) == -3
    assert _status("tdc_update", FAKE, FAKE, None, ctypes.c_void_p(0x900000), 64, FAKE, FAKE, 0, None) == -5
    assert _status("tdc_apply", FAKE, ctypes.c_void_p(0x10040), ctypes.c_void_p(0x10040), 64, None, None, 0, None) == -7
    assert _status("tdc_apply", FAKE, ctypes.c_void_p(0x900000), ctypes.c_void_p(0x10020), 64, None, None, 0, None) == -7
    assert _status("block_gamma", FAKE, FAKE, -1, FAKE, FAKE, 1 << 20, None) == -1
    assert _status("block_gamma", FAKE, FAKE, 64, None, FAKE, 1 << 20, None) == -1


def test_noalloc_scratch_limit():
    """qlinear_int8_noalloc refuses a shape whose workspace exceeds the static
    scratch before it touches a device, and returns qlinear_int8's status for
    a rejected shape (its workspace size is then 0)."""
    assert qa.NOALLOC_SCRATCH_BYTES == 64 << 20
    big = (256, 131072, 16384)          # 128 MiB of weight-scale copies
    assert qa.qlinear_workspace(qa.INT8, *big) > qa.NOALLOC_SCRATCH_BYTES
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, None]
    assert _status("qlinear_int8_noalloc", *args, *big, None, FAKE, big[1], 0, 0, None) == -8
    assert _status("qlinear_int8_noalloc", *args, 4, 64, 24, None, FAKE, 64, 0, 0, None) == -2
    assert qa.qlinear_workspace(qa.INT8, 4, 64, 24) == 0
    assert qa.qlinear_workspace(qa.INT8, 4, 64, 1 << 23) == 0
    assert _status("qlinear_int8_noalloc", *args, 4, 64, 1 << 23, None, FAKE, 64, 0, 0, None) == -2
    # the CogVideoX-2B and -5B block linears at 17776 tokens fit
    for n, k in ((5760, 1920), (7680, 1920), (1920, 7680), (9216, 3072), (3072, 12288),
                 (12288, 3072)):
        assert 0 < qa.qlinear_workspace(qa.INT8, 17776, n, k) <= qa.NOALLOC_SCRATCH_BYTES


def test_convert_check_validation():
    # the test-only conversion entry point rejects bad arguments before any launch
    assert _status("qa_test_convert", 3, 0, 16, FAKE, None) == -1
    assert _status("qa_test_convert", 0, 0, -1, FAKE, None) == -1
    assert _status("qa_test_convert", 0, 0xFFFFFFF0, 17, FAKE, None) == -1
    assert _status("qa_test_convert", 0, 0, 16, None, None) == -1
    assert _status("qa_test_convert", 2, 0, 16, ctypes.c_void_p(0x10001), None) == -3
    assert _status("qa_test_convert", 1, 0x7F7FFFF0, 17, FAKE, None) == -1   # past the finite range
    assert _status("qa_test_convert", 1, 0x80000000, 1, FAKE, None) == -1    # negative scale
    assert _status("qa_test_convert", 0, 5, 0, FAKE, None) == 0              # nothing to do


def test_routed_and_stage_validation():
    # act_quant_routed: route byte and both formats' buffers required; shapes
    # and alignment as act_quant; outputs must not overlap each other
    A = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(8)]
    ok = [A[0], A[1], 64, 256, 256, A[2], A[3], A[4], 1, None, 0, A[5], A[6], None]
    assert _status("act_quant_routed", None, *ok[1:]) == -1
    bad_k = list(ok); bad_k[3] = 24; bad_k[4] = 24
    assert _status("act_quant_routed", *bad_k) == -2
    no_ws = list(ok); no_ws[8] = 0
    assert _status("act_quant_routed", *no_ws) == -5
    alias = list(ok); alias[11] = A[2]                              # q8 on q4
    assert _status("act_quant_routed", *alias) == -7
    # ring calls: the slots must not overlap each other or the other buffers
    assert _status("tdc_update_ring", None, A[0], A[1], A[2], A[3], 64, A[4], A[5], 1 << 20,
                   None) == -1
    assert _status("tdc_update_ring", A[6], A[0], A[1], A[2], A[2], 64, A[4], A[5], 1 << 20,
                   None) == -7
    assert _status("tdc_apply_ring", A[6], A[0], A[2], A[3], A[2], 64, None, None, None, 0,
                   None) == -7
    # stage A/B: design and sizes checked before any launch
    assert _status("qa_test_stage_ab", 3, 1, 1, A[0], A[1], None) == -1
    assert _status("qa_test_stage_ab", 0, 1, 0, A[0], A[1], None) == -1
    assert _status("qa_test_stage_ab", 0, 1, 1, ctypes.c_void_p(0x100002), A[1], None) == -3


def test_routed_linear_validation():
    # qlinear_routed: route byte and both formats' operands required; bf16
    # staged output only; K % 16; alignment; the NVFP4 workspace at least;
    # the output must not overlap operands, workspace or the route byte
    A = [ctypes.c_void_p(0x1000000 * (i + 1)) for i in range(16)]
    M, N, K = 64, 256, 256
    ok = [A[0], A[1], A[2], A[3], A[4], A[5], A[6], A[7], A[8], A[9], M, N, K, None, A[10], N, 0,
          None, A[11], 1 << 24, None]
    assert qa.lib().qlinear_routed_workspace(M, N, K) > 0
    assert qa.lib().qlinear_routed_workspace(M, N, 24) == 0
    for i in range(10):                                   # any missing operand
        bad = list(ok); bad[i] = None
        assert _status("qlinear_routed", *bad) == -1, i
    bad = list(ok); bad[12] = 24
    assert _status("qlinear_routed", *bad) == -2           # K % 16
    bad = list(ok); bad[15] = N - 1
    assert _status("qlinear_routed", *bad) == -2           # ldy < N
    bad = list(ok); bad[9] = ctypes.c_void_p(0x1000000 * 10 + 16)
    assert _status("qlinear_routed", *bad) == -3           # w8 256-byte aligned
    bad = list(ok); bad[14] = ctypes.c_void_p(0x1000000 * 11 + 2)
    assert _status("qlinear_routed", *bad) == -4           # y not 16-byte aligned: unsupported
    bad = list(ok); bad[19] = 0
    assert _status("qlinear_routed", *bad) == -5           # no workspace
    bad = list(ok); bad[14] = A[1]
    assert _status("qlinear_routed", *bad) == -7           # y on a_q4
    bad = list(ok); bad[0] = ctypes.c_void_p(0x1000000 * 11 + 64)
    assert _status("qlinear_routed", *bad) == -7           # route byte inside y


def test_strerror_covers_codes():
    for s in range(-8, 1):
        assert qa.strerror(s) != "unknown status"


def test_dmpq_mask_matches_oracle():
    rng = np.random.default_rng(0)
    L, J = 42, 4
    g = rng.uniform(0, 0.2, L)
    alpha = rng.uniform(0.5, 1.5, L * J).astype(np.float32)
    beta = rng.uniform(0, 0.02, L * J).astype(np.float32)
    for tau in (0.05, 0.1, 0.15):
        np.testing.assert_array_equal(qa.dmpq_mask(g, alpha, beta, tau, L, J),
                                      T.dmpq_mask(g, alpha, beta, tau, J))
    np.testing.assert_array_equal(qa.dmpq_mask(None, alpha, beta, 0.1, L, J),
                                  T.dmpq_mask(None, alpha, beta, 0.1, J))
    # the worked tie: p == tau -> NVFP4
    p = float(np.float32(1.0)) * 0.125 + float(np.float32(2.0 ** -7))
    assert qa.dmpq_mask([0.125], [1.0], [2.0 ** -7], p, 1, 1)[0] == 0
    assert qa.dmpq_mask([0.125], [1.0], [2.0 ** -7], 0.125, 1, 1)[0] == 1


def test_tdc_decide_matches_oracle():
    rng = np.random.default_rng(1)
    d = rng.uniform(0, 0.1, 30)
    d[3] = 0.05
    c = rng.integers(0, 2, 30).astype(np.uint8)
    for t in range(4):
        np.testing.assert_array_equal(qa.tdc_decide(t, d, c, 0.05), T.tdc_decide(t, d, c, 0.05))


def test_sum_helpers():
    assert qa.gamma_from_sums([0.0, 0.0]) == 0.0
    assert qa.gamma_from_sums([1.0, 0.0]) == float("inf")
    assert qa.rel_l2_from_sums([0, 0, 6.25 * 2.0 ** -10, 6.25]) == 0.03125


def test_dmpq_fit_matches_oracle():
    # host function: the long-double least squares equals the oracle's exact
    # rational fit rounded to float32, pairs (Gamma_{t-1}, E_rel_t)
    from oracle import tdc as T
    rng = np.random.default_rng(21)
    Tn, L, J = 9, 4, 3
    g = rng.uniform(0.0, 0.3, (Tn, L))
    e = np.repeat(g, J, axis=1) * 0.7 + 0.02 + 0.005 * rng.standard_normal((Tn, L * J))
    e = np.roll(e, 1, axis=0)                  # E_rel_t follows Gamma_{t-1}
    e[0] = np.nan
    e[4, 5] = np.inf                           # dropped pair
    g[6, 2] = np.nan                           # drops (Gamma_6, E_rel_7) of block 2
    a, b = qa.dmpq_fit(g, e, J)
    ao, bo = T.calibrate(g, e, J)
    assert np.array_equal(a, ao) and np.array_equal(b, bo), (a - ao, b - bo)


def test_dmpq_fit_degenerate_and_validation():
    g = np.full((5, 1), 0.1)                   # one x value: alpha 0, beta = mean
    e = np.array([[np.nan], [1.0], [2.0], [3.0], [6.0]])
    a, b = qa.dmpq_fit(g, e, 1)
    assert a[0] == 0.0 and b[0] == 3.0
    a, b = qa.dmpq_fit(np.zeros((1, 2)), np.zeros((1, 2)), 1)   # T = 1: no pairs
    assert np.all(a == 0) and np.all(b == 0)
    f = qa.lib().dmpq_fit
    out = np.zeros(4, np.float32)
    assert f(None, None, 3, 2, 0, out.ctypes.data, out.ctypes.data) == -1   # J <= 0
    assert f(None, None, 3, 2, 1, out.ctypes.data, out.ctypes.data) == -1   # arrays needed
    assert f(None, None, 0, 2, 1, out.ctypes.data, out.ctypes.data) == 0    # T = 0: nothing to read
    assert qa.rel_err_from_sums(np.array([1.0, 25.0])) == 0.2
    assert qa.rel_err_from_sums(np.array([0.0, 0.0])) == 0.0
    assert qa.rel_err_from_sums(np.array([1.0, 0.0])) == float("inf")


def test_rel_err_validation():
    assert _status("rel_err", FAKE, FAKE, 64, None, FAKE, 1 << 20, None) == -1
    assert _status("rel_err", FAKE, FAKE, 64, FAKE, None, 0, None) == -5
    assert _status("rel_err", FAKE, FAKE_ODD, 64, FAKE, FAKE, 1 << 20, None) == -3


def test_quantized_output_validation():
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]
    yq, ys = ctypes.c_void_p(0x900000), ctypes.c_void_p(0xA00000)
    big = 1 << 40
    # N must be a multiple of 16 (whole NVFP4 groups)
    assert _status("qlinear_nvfp4_q", *ok, 4, 24, 16, None, 0, FAKE, yq, ys, FAKE, big, None) == -2
    # a tensor scale and both outputs are required; codes 16-byte aligned
    assert _status("qlinear_nvfp4_q", *ok, 4, 32, 16, None, 0, None, yq, ys, FAKE, big, None) == -1
    assert _status("qlinear_nvfp4_q", *ok, 4, 32, 16, None, 0, FAKE, None, ys, FAKE, big, None) == -1
    assert _status("qlinear_nvfp4_q", *ok, 4, 32, 16, None, 0, FAKE, ctypes.c_void_p(0x900004), ys,
                   FAKE, big, None) == -3
    assert _status("qlinear_nvfp4_q", *ok, 4, 32, 16, None, 7, FAKE, yq, ys, FAKE, big, None) == -1
    # codes overlapping the scales
    assert _status("qlinear_nvfp4_q", *ok, 4, 32, 16, None, 0, FAKE, yq, ctypes.c_void_p(0x900008),
                   FAKE, big, None) == -7
    assert _status("qlinear_int8_q", *ok[:5], None, 4, 32, 16, None, 0, FAKE, yq, ys, FAKE, 0, None) == -5


def test_cosine_helpers_match_oracle():
    from oracle import tdc as T
    rng = np.random.default_rng(9)
    for _ in range(20):
        s = np.array([rng.standard_normal(), abs(rng.standard_normal()), abs(rng.standard_normal())])
        assert qa.cosine_from_sums(s) == T.cosine(*s)
    assert qa.cosine_from_sums(np.array([1.0, 0.0, 4.0])) == 0.0
    for t in (0, 1, 2, 7):
        c = rng.uniform(0.8, 1.0, 9)
        cp = rng.integers(0, 2, 9)
        np.testing.assert_array_equal(qa.tdc_decide_cos(t, c, cp, 0.9),
                                      T.tdc_decide_cos(t, c, cp, 0.9))
    assert _status("delta_cosine", FAKE, FAKE, 64, None, FAKE, 1 << 20, None) == -1
    assert _status("delta_cosine", FAKE, FAKE, 64, FAKE, None, 0, None) == -5


def test_step_control_validation():
    # a gate needs bits; clearing takes none; decisions check shapes,
    # pointers and alignment before any launch
    assert _status("qa_set_gate", FAKE, 0) == -1
    assert _status("qa_set_gate", None, 0) == 0
    ok = [FAKE, FAKE, FAKE, 0.5, 0.05]
    st = [FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None]
    assert _status("qa_decide_step", *ok, 0, 4, *st) == -2
    assert _status("qa_decide_step", *ok, 4, 0, *st) == -2
    assert _status("qa_decide_step", None, *ok[1:], 4, 4, *st) == -1
    assert _status("qa_decide_step", *ok, 4, 4, FAKE, FAKE, FAKE, None, FAKE, None, None, None) == -1
    assert _status("qa_decide_step", ctypes.c_void_p(FAKE.value + 4), *ok[1:], 4, 4, *st) == -3


def test_amax_output_validation():
    # the |max| output needs a target, 4-byte alignment and the staged bf16
    # epilogue (16-byte aligned y, ldy % 4 == 0); it may not alias y or ws
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]
    y = ctypes.c_void_p(0x900000)
    assert _status("qlinear_nvfp4_amax", *ok, 4, 4, 16, None, y, 4, 0, None, FAKE, 1 << 20, None) == -1
    assert _status("qlinear_nvfp4_amax", *ok, 4, 4, 16, None, y, 4, 0, ctypes.c_void_p(0xA00002),
                   FAKE, 1 << 20, None) == -3
    assert _status("qlinear_nvfp4_amax", *ok, 4, 4, 16, None, ctypes.c_void_p(0x900008), 4, 0,
                   ctypes.c_void_p(0xA00000), FAKE, 1 << 20, None) == -4
    assert _status("qlinear_int8_amax", *ok[:5], None, 4, 4, 16, None, y, 6, 0, ctypes.c_void_p(0xA00000),
                   FAKE, 1 << 20, None) == -4
    assert _status("qlinear_int8_amax", *ok[:5], None, 4, 4, 16, None, y, 4, 0, ctypes.c_void_p(0x900004),
                   FAKE, 1 << 20, None) == -7


def test_shape_limits():
    # 32-bit offsets of a tile's operand rows: K < 2^23; rows below 2^26
    w = ctypes.c_void_p(0x900000)
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]
    big = 1 << 40
    for M, N, K in ((4, 4, 1 << 23), (1 << 26, 4, 16), (4, 1 << 26, 16)):
        assert _status("qlinear_nvfp4", *ok, M, N, K, None, w, N, 0, 0, FAKE, big, None) == -2
        assert _status("qlinear_int8", *ok[:5], None, M, N, K, None, w, N, 0, 0, FAKE, big,
                       None) == -2
    assert _status("act_quant", 1, FAKE, 4, 1 << 23, 1 << 23, w, FAKE, None, 0, None, 0,
                   None) == -2
    assert _status("act_quant", 1, FAKE, 1 << 26, 16, 16, w, FAKE, None, 0, None, 0, None) == -2
    # the largest accepted sizes pass the shape checks (and fail later, on
    # the workspace, without touching memory)
    assert _status("qlinear_nvfp4", *ok, 4, 4, (1 << 23) - 16, None, w, 4, 0, 0, FAKE, 0,
                   None) == -5


def test_int8_planes_validation_and_size():
    w8 = ctypes.c_void_p(0x100000)
    need = qa.int8_weight_planes_bytes(5760, 1920)
    r256 = lambda b: (b + 255) // 256 * 256
    # 45 weight-row tiles of 128 x 30 units of 64, 16 KB each (two digit
    # planes of 128 rows x 64 bytes), then one float per padded row and the
    # irregular-row counter
    assert need == r256(45 * 30 * 16384) + r256(45 * 128 * 4) + 256
    assert qa.int8_weight_planes_bytes(4, 24) == 0
    cnt = ctypes.c_int64(0)
    pcnt = ctypes.addressof(cnt)
    assert _status("int8_weight_planes", None, FAKE, 4, 16, w8, 1 << 20, pcnt, None) == -1
    assert _status("int8_weight_planes", FAKE, FAKE, 4, 24, w8, 1 << 20, pcnt, None) == -2
    assert _status("int8_weight_planes", FAKE, FAKE, 4, 16, ctypes.c_void_p(0x100010), 1 << 20,
                   pcnt, None) == -3
    assert _status("int8_weight_planes", FAKE, FAKE, 4, 16, w8, 64, pcnt, None) == -5
    assert _status("int8_weight_planes", FAKE, FAKE, 4, 16, FAKE, 1 << 20, pcnt, None) == -7


def test_int8_acc_and_w8_validation():
    w8 = ctypes.c_void_p(0x100000)
    y = ctypes.c_void_p(0x900000)
    assert _status("qlinear_int8_acc", None, w8, 4, 4, 16, y, y, None) == -1
    assert _status("qlinear_int8_acc", FAKE, w8, 4, 4, 1 << 17, FAKE, FAKE, None) == -2
    assert _status("qlinear_int8_acc", FAKE, ctypes.c_void_p(0x100010), 4, 4, 16,
                   ctypes.c_void_p(0x2000000), ctypes.c_void_p(0x3000000), None) == -3
    assert _status("qlinear_int8_acc", FAKE, w8, 4, 4, 16, ctypes.c_void_p(0x2000000),
                   ctypes.c_void_p(0x2000010), None) == -7
    # with w8 the NVFP4 weight pointers may be null and no workspace is needed
    assert _status("qlinear_int8", FAKE, FAKE, None, None, FAKE, ctypes.c_void_p(0x100010), 4, 4,
                   16, None, y, 4, 0, 0, None, 0, None) == -3
    assert _status("qlinear_int8", FAKE, FAKE, None, None, FAKE, None, 4, 4, 16, None, y, 4, 0,
                   0, None, 0, None) == -1
    # the layer call takes w8 for INT8 only
    assert _status("qlinear", 0, FAKE, 16, FAKE, 0, FAKE, FAKE, FAKE, w8, 4, 4, 16, None, y, 4,
                   0, 0, FAKE, 1 << 30, None) == -1
