"""qlinear_int8_noalloc (the INT8 linear with its workspace in the library's
static device array) against qlinear_int8 given a workspace of its own:
the same kernels, so the outputs must agree bit for bit.  Two calls in a
row, the second on a smaller input that also splits along K, so it runs
over the partial sums the first call left in the array; then a call on the
fp16-MFMA kernel (no digit planes), and the outputs also against the
oracle's exact integer form."""
import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q
from tests._gpu import dev, host, sample_rows, torch

pytestmark = pytest.mark.gpu


def _qa():
    import mixed_precision_quantized_act_amd as qa
    return qa


def _operands(M, N, K, seed):
    qa = _qa()
    x = synth.activations(seed, M, K, "normal", min(4, K // 16), 20.0)
    w = synth.weight(seed, 0, N, K)
    a = Q.int8_encode(x)
    wq = Q.nvfp4_encode(w)
    w8 = qa.empty_int8_planes(N, K)
    qa.int8_weight_planes(dev(wq[0]), dev(wq[1]), w8, N, K)
    ops = dict(a_q=dev(a[0]), a_s=dev(a[1]), w_q=dev(wq[0]), w_s=dev(wq[1]),
               w_ts=dev(np.array([wq[2]], np.float32)), w8=w8)
    return a, wq, ops


def _pair(ops, M, N, K, out_f32, gelu, bias, use_w8):
    """(noalloc output, qlinear_int8 output) on the same operands."""
    qa, t = _qa(), torch()
    dt = t.float32 if out_f32 else t.bfloat16
    kw = dict(bias=bias, out=qa.OUT_F32 if out_f32 else qa.OUT_BF16,
              epi=qa.EPI_GELU_TANH if gelu else qa.EPI_NONE)
    w8 = ops["w8"] if use_w8 else None
    y0 = t.full((M, N), float("nan"), dtype=dt, device="cuda")
    qa.qlinear_int8_noalloc(ops["a_q"], ops["a_s"], ops["w_q"], ops["w_s"], ops["w_ts"], y0, M,
                            N, K, w8=w8, **kw)
    t.cuda.synchronize()
    y1 = t.full((M, N), float("nan"), dtype=dt, device="cuda")
    ws = qa.workspace(qa.qlinear_workspace(qa.INT8, M, N, K))
    qa.qlinear_int8(ops["a_q"], ops["a_s"], ops["w_q"], ops["w_s"], ops["w_ts"], y1, M, N, K,
                    ws=ws, w8=w8, **kw)
    t.cuda.synchronize()
    return host(y0), host(y1)


def _exact(a, wq, rows):
    integer, X, regular = G.int8_weight_integers(wq[0], wq[1])
    assert regular.all()
    hi, lo = G.int8_digits(integer)
    H, L = G.int8_accumulators(a[0][rows], hi, lo)
    return G.int8_linear_from_sums(H, L, X, a[1][rows], wq[2])


def test_noalloc_two_calls_then_fp16_kernel():
    qa = _qa()
    # 3 x 6 = 18 tiles split 4 ways along K (18 MB of partials), then a
    # smaller 2 x 3 = 6-tile call, also split, over what the first left
    shapes = [(600, 700, 3840, True, False), (300, 384, 3840, False, True)]
    for i, (M, N, K, out_f32, gelu) in enumerate(shapes):
        print(f"[noalloc] call {i}: M={M} N={N} K={K} w8", flush=True)
        # beyond 1 MiB: the K split's int32 partials (256 KB per tile slice)
        assert (1 << 20) < qa.qlinear_workspace(qa.INT8, M, N, K) <= qa.NOALLOC_SCRATCH_BYTES
        a, wq, ops = _operands(M, N, K, seed=60 + i)
        bias = None if out_f32 else dev(F.f64_to_bf16_rne(
            np.random.default_rng(70 + i).normal(0, 0.5, N)))
        y0, y1 = _pair(ops, M, N, K, out_f32, gelu, bias, True)
        np.testing.assert_array_equal(y0, y1)
        assert np.isfinite(y0.astype(np.float64) if out_f32 else F.bf16_to_f64(y0)).all()
        if out_f32:
            rows = sample_rows(M, 64, seed=8)
            Y = _exact(a, wq, rows)
            got = y0[rows].astype(np.float64)
            assert np.all(np.abs(got - Y) <= 4 * 2.0 ** -24 * np.abs(Y))
    # the fp16-MFMA INT8 kernel (no digit planes) through the same scratch
    M, N, K = 257, 300, 1920
    print(f"[noalloc] call 2: M={M} N={N} K={K} fp16 kernel", flush=True)
    _, _, ops = _operands(M, N, K, seed=62)
    y0, y1 = _pair(ops, M, N, K, True, False, None, False)
    np.testing.assert_array_equal(y0, y1)
    assert np.isfinite(y0).all()


def test_noalloc_refuses_beyond_scratch():
    qa, t = _qa(), torch()
    M, N, K = 256, 131072, 16384          # 128 MiB of weight-scale copies
    assert qa.qlinear_workspace(qa.INT8, M, N, K) > qa.NOALLOC_SCRATCH_BYTES
    a_q = t.zeros((16,), dtype=t.int8, device="cuda")
    f = t.ones((16,), dtype=t.float32, device="cuda")
    u = t.zeros((16,), dtype=t.uint8, device="cuda")
    y = t.zeros((16,), dtype=t.bfloat16, device="cuda")
    with pytest.raises(qa.QactError) as e:
        qa.qlinear_int8_noalloc(a_q, f, u, u, f, y, M, N, K, ldy=N)
    assert e.value.status == -8
