"""GPU parity of act_quant (NVFP4 and INT8): codes, scales and the tensor
scale are compared bit for bit with the oracle on the same bf16 bytes."""
import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import quant as Q
from tests._gpu import dev, host, sample_rows, torch

pytestmark = pytest.mark.gpu


def _qa():
    import mixed_precision_quantized_act_amd as qa
    return qa


def gpu_nvfp4(x, tscale=None, ldx=None):
    qa, t = _qa(), torch()
    M, K = x.shape[0], (x.shape[1] if ldx is None else ldx[1])
    xd = dev(x)
    codes, scales, ts = qa.empty_nvfp4(M, K)
    flags = 0
    if tscale is not None:
        ts.fill_(float(tscale))
        flags = qa.TSCALE_GIVEN
    ws = qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, K))
    qa.act_quant(qa.NVFP4, xd, codes, scales, ts, flags, ws, M=M, K=K)
    t.cuda.synchronize()
    return host(codes), host(scales), np.float32(host(ts)[0])


def gpu_int8(x, K=None):
    qa, t = _qa(), torch()
    M = x.shape[0]
    K = x.shape[1] if K is None else K
    q, s = qa.empty_int8_act(M, K)
    qa.act_quant(qa.INT8, dev(x), q, s, M=M, K=K)
    t.cuda.synchronize()
    return host(q), host(s)


def test_nvfp4_worked_group():
    x = F.f64_to_bf16_rne(np.array([[2688] + [0] * 15 + [0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2.5,
                                                        3.5, 5, 5.5, 6, -.125, -1.75, -5]]))
    c, s, ts = gpu_nvfp4(x)
    assert ts == 1.0
    assert s.ravel().tolist() == [0x7E, 0x38]
    assert c.ravel().tolist() == [0x07] + [0] * 7 + [0x00, 0x21, 0x22, 0x43, 0x64, 0x76, 0x87, 0xEC]


@pytest.mark.parametrize("M,K", [(256, 256), (1, 16), (37, 48), (300, 1920), (5, 7680)])
def test_nvfp4_matches_oracle(M, K):
    x = synth.activations(1, M, K, "normal", min(4, K), 20.0)
    c, s, ts = gpu_nvfp4(x)
    oc, os_, ots = Q.nvfp4_encode(x)
    assert ts == ots
    np.testing.assert_array_equal(s, os_)
    np.testing.assert_array_equal(c, oc)


def test_nvfp4_given_scale_and_ld():
    x = synth.activations(1, 64, 320, "t3")
    sub = np.ascontiguousarray(x[:, :256])
    c, s, ts = gpu_nvfp4_ld(x, 256)
    oc, os_, _ = Q.nvfp4_encode(sub, tscale=np.float32(0.0123))
    np.testing.assert_array_equal(s, os_)
    np.testing.assert_array_equal(c, oc)


def gpu_nvfp4_ld(x, K):
    qa, t = _qa(), torch()
    M = x.shape[0]
    codes, scales, ts = qa.empty_nvfp4(M, K)
    ts.fill_(0.0123)
    qa.act_quant(qa.NVFP4, dev(x), codes, scales, ts, qa.TSCALE_GIVEN, None, M=M, K=K,
                 ldx=x.shape[1])
    t.cuda.synchronize()
    return host(codes), host(scales), host(ts)[0]


def test_nvfp4_all_bf16_values():
    # every finite bf16 pattern of magnitude below 2^100, 16 per group, with
    # groups drawn in a fixed shuffled order; tensor scale given so that the
    # group scales span the E4M3 range including subnormal codes
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f64(bits)
    keep = bits[np.isfinite(v) & (np.abs(v) < 2.0 ** 100)]
    keep = keep[: len(keep) // 16 * 16]
    perm = np.random.default_rng(0).permutation(len(keep))
    x = keep[perm].reshape(-1, 16 * 16)
    for ts in (np.float32(2.0 ** 90), np.float32(1e-3), np.float32(3.7)):
        qa, t = _qa(), torch()
        M, K = x.shape
        codes, scales, tsd = qa.empty_nvfp4(M, K)
        tsd.fill_(float(ts))
        qa.act_quant(qa.NVFP4, dev(x), codes, scales, tsd, qa.TSCALE_GIVEN, None)
        t.cuda.synchronize()
        oc, os_, _ = Q.nvfp4_encode(x, tscale=ts)
        np.testing.assert_array_equal(host(scales), os_)
        np.testing.assert_array_equal(host(codes), oc)


def test_nvfp4_zero_and_negative_zero():
    x = np.zeros((3, 32), np.uint16)
    x[1, 3] = 0x8000
    c, s, ts = gpu_nvfp4(x)
    oc, os_, ots = Q.nvfp4_encode(x)
    assert ts == ots == 0
    np.testing.assert_array_equal(c, oc)
    np.testing.assert_array_equal(s, os_)


def test_nvfp4_full_qkv_shape_sampled_rows():
    x, _ = synth.linear_case(2)
    c, s, ts = gpu_nvfp4(x)
    assert ts == Q.nvfp4_tensor_scale(x)
    rows = sample_rows(x.shape[0], 512, seed=1)
    oc, os_, _ = Q.nvfp4_encode(x[rows], tscale=ts)
    np.testing.assert_array_equal(s[rows], os_)
    np.testing.assert_array_equal(c[rows], oc)


@pytest.mark.parametrize("M,K", [(256, 256), (1, 16), (37, 48), (300, 1920), (9, 7680)])
def test_int8_matches_oracle(M, K):
    x = synth.activations(1, M, K, "normal", min(4, K), 20.0)
    q, s = gpu_int8(x)
    oq, os_ = Q.int8_encode(x)
    np.testing.assert_array_equal(s, os_)
    np.testing.assert_array_equal(q, oq)


def test_int8_all_bf16_values():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f64(bits)
    keep = bits[np.isfinite(v)]
    keep = keep[: len(keep) // 64 * 64]
    x = keep[np.random.default_rng(1).permutation(len(keep))].reshape(-1, 64)
    q, s = gpu_int8(x)
    oq, os_ = Q.int8_encode(x)
    np.testing.assert_array_equal(s, os_)
    np.testing.assert_array_equal(q, oq)


def test_int8_full_qkv_shape_sampled_rows():
    x, _ = synth.linear_case(2)
    q, s = gpu_int8(x)
    rows = sample_rows(x.shape[0], 1024, seed=2)
    oq, os_ = Q.int8_encode(x[rows])
    np.testing.assert_array_equal(s[rows], os_)
    np.testing.assert_array_equal(q[rows], oq)


def test_deterministic_repeat():
    x = synth.activations(3, 512, 1920, "t3")
    a = gpu_nvfp4(x)
    b = gpu_nvfp4(x)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)



def _nvfp4_with(x, M, K, ldx=None):
    """act_quant NVFP4 of the first K columns of x (rows of ldx elements);
    returns codes, scales, tensor scale (host)."""
    qa, t = _qa(), torch()
    codes, scales, ts = qa.empty_nvfp4(M, K)
    ws = qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, K))
    qa.act_quant(qa.NVFP4, dev(x), codes, scales, ts, 0, ws, M=M, K=K,
                 ldx=K if ldx is None else ldx)
    t.cuda.synchronize()
    return host(codes), host(scales), np.float32(host(ts)[0])


def test_nvfp4_strided_equals_contiguous_full_shape():
    # the QKV activation contiguous (one flat tensor-max sweep) and at a
    # padded row stride (row-by-row sweep) whose padding holds a huge value:
    # the same bytes, the padding never entering the tensor maximum
    x, _ = synth.linear_case(2)
    M, K = x.shape
    one = _nvfp4_with(x, M, K)
    pad = np.zeros((M, K + 16), np.uint16)
    pad[:, :K] = x
    pad[:, K:] = 0x7F7F
    two = _nvfp4_with(pad, M, K, ldx=K + 16)
    for a, b in zip(one, two):
        np.testing.assert_array_equal(a, b)
    assert one[2] == Q.nvfp4_tensor_scale(x)


def test_nvfp4_5b_hidden_shape_sampled_rows():
    # a CogVideoX-5B block input (17776 x 3072, 19 outlier channels x30)
    M, K = 17776, 3072
    x = synth.activations(5, M, K, "normal", 19, 30.0)
    c, s, ts = _nvfp4_with(x, M, K)
    assert ts == Q.nvfp4_tensor_scale(x)
    rows = sample_rows(M, 256, seed=3)
    oc, os_, _ = Q.nvfp4_encode(x[rows], tscale=ts)
    np.testing.assert_array_equal(s[rows], os_)
    np.testing.assert_array_equal(c[rows], oc)
