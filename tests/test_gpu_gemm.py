"""GPU parity of the quantized linears.  Outputs: relative Frobenius error
<= 1e-3 against the float64 oracle rounded to the output type (the
tolerance the method's checker states); float32 outputs also element by
element within the float32-accumulation bound (K + 3) 2^-24 sum_k |a_k w_k|
of exactly dequantized operands, and bit-exact where every partial sum is
exact in float32.  Operands are quantized by the oracle, so the GEMM is
isolated."""
import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q
from tests._gpu import dev, host, rel_fro, sample_rows, torch

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _qa():
    import mixed_precision_quantized_act_amd as qa
    return qa


def _round_ref(y, out_f32):
    if out_f32:
        return y.astype(np.float32).astype(np.float64)
    return F.bf16_to_f64(F.f64_to_bf16_rne(y))


def _out_host(y, out_f32):
    return host(y).astype(np.float64) if out_f32 else F.bf16_to_f64(host(y))


def run_nvfp4(a, w, M, N, K, bias=None, out_f32=False, gelu=False, y_rows=None):
    qa, t = _qa(), torch()
    y = t.empty((M, N), dtype=t.float32 if out_f32 else t.bfloat16, device="cuda")
    ws = qa.workspace(qa.qlinear_workspace(qa.NVFP4, M, N, K))
    qa.qlinear_nvfp4(dev(a[0]), dev(a[1]), dev(np.array([a[2]], np.float32)),
                     dev(w[0]), dev(w[1]), dev(np.array([w[2]], np.float32)), y, M, N, K,
                     bias=None if bias is None else dev(bias),
                     out=qa.OUT_F32 if out_f32 else qa.OUT_BF16,
                     epi=qa.EPI_GELU_TANH if gelu else qa.EPI_NONE, ws=ws)
    t.cuda.synchronize()
    return _out_host(y, out_f32)


def run_int8(a, w, M, N, K, bias=None, out_f32=False, gelu=False):
    qa, t = _qa(), torch()
    y = t.empty((M, N), dtype=t.float32 if out_f32 else t.bfloat16, device="cuda")
    ws = qa.workspace(qa.qlinear_workspace(qa.INT8, M, N, K))
    qa.qlinear_int8(dev(a[0]), dev(a[1]), dev(w[0]), dev(w[1]),
                    dev(np.array([w[2]], np.float32)), y, M, N, K,
                    bias=None if bias is None else dev(bias),
                    out=qa.OUT_F32 if out_f32 else qa.OUT_BF16,
                    epi=qa.EPI_GELU_TANH if gelu else qa.EPI_NONE, ws=ws)
    t.cuda.synchronize()
    return _out_host(y, out_f32)


def _case(M, N, K, seed, dist="normal"):
    x = synth.activations(seed, M, K, dist, min(4, K // 16), 20.0 if dist == "normal" else 1.0)
    w = synth.weight(seed, 0, N, K)
    return x, w


SHAPES = [(256, 256, 256), (1, 16, 16), (300, 200, 48), (257, 300, 80), (77, 90, 112),
          (513, 257, 96), (64, 5760, 1920), (130, 7680, 1920), (70, 1920, 7680)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("out_f32", [False, True])
def test_nvfp4_linear(M, N, K, out_f32):
    x, w = _case(M, N, K, seed=11)
    a, wq = Q.nvfp4_encode(x), Q.nvfp4_encode(w)
    ref = G.linear_ref(Q.nvfp4_decode(*a), Q.nvfp4_decode(*wq))
    y = run_nvfp4(a, wq, M, N, K, out_f32=out_f32)
    assert rel_fro(y, _round_ref(ref, out_f32)) <= TOL


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("out_f32", [False, True])
def test_int8_linear(M, N, K, out_f32):
    x, w = _case(M, N, K, seed=12)
    a, wq = Q.int8_encode(x), Q.nvfp4_encode(w)
    ref = G.linear_ref(Q.int8_decode(*a), Q.nvfp4_decode(*wq))
    y = run_int8(a, wq, M, N, K, out_f32=out_f32)
    assert rel_fro(y, _round_ref(ref, out_f32)) <= TOL


def _elementwise_bound(a_deq, w_deq, K):
    # float32 accumulation of K exact products, then at most two float32
    # scalings: |y - exact| <= (K + 3) 2^-24 sum_k |a_k w_k|
    return (K + 3) * 2.0 ** -24 * (np.abs(a_deq) @ np.abs(w_deq).T) + 1e-300


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (300, 200, 48), (130, 640, 1920),
                                   (33, 96, 7680)])
@pytest.mark.parametrize("path", ["nvfp4", "int8"])
def test_f32_output_elementwise_bound(M, N, K, path):
    x, w = _case(M, N, K, seed=13)
    wq = Q.nvfp4_encode(w)
    wd = Q.nvfp4_decode(*wq)
    if path == "nvfp4":
        a = Q.nvfp4_encode(x)
        ad = Q.nvfp4_decode(*a)
        y = run_nvfp4(a, wq, M, N, K, out_f32=True)
    else:
        a = Q.int8_encode(x)
        ad = Q.int8_decode(*a)
        y = run_int8(a, wq, M, N, K, out_f32=True)
    ref = G.linear_ref(ad, wd)
    err = np.abs(y - ref)
    bound = _elementwise_bound(ad, wd, K)
    assert np.all(err <= bound), float(np.max(err / bound))


def _run_ws(path, a, wq, M, N, K, split, bias=None, gelu=False):
    """float32 output with the full workspace (the last round of tiles split
    along K) or one byte short of it (every tile whole)."""
    qa, t = _qa(), torch()
    fmt = qa.NVFP4 if path == "nvfp4" else qa.INT8
    full = qa.qlinear_workspace(fmt, M, N, K)
    ws = qa.workspace(full)
    if not split:
        ws = ws[:full - 1]
    y = t.empty((M, N), dtype=t.float32, device="cuda")
    b = None if bias is None else dev(bias)
    epi = qa.EPI_GELU_TANH if gelu else qa.EPI_NONE
    w3 = (dev(wq[0]), dev(wq[1]), dev(np.array([wq[2]], np.float32)))
    if path == "nvfp4":
        qa.qlinear_nvfp4(dev(a[0]), dev(a[1]), dev(np.array([a[2]], np.float32)), *w3, y, M, N, K,
                         bias=b, out=qa.OUT_F32, epi=epi, ws=ws)
    else:
        qa.qlinear_int8(dev(a[0]), dev(a[1]), *w3, y, M, N, K, bias=b, out=qa.OUT_F32, epi=epi,
                        ws=ws)
    t.cuda.synchronize()
    return host(y).astype(np.float64)


# (M, N, K): 9 tiles in 4 slices of 15 units; 6 tiles in 4 slices of 13,
# 13, 13 and 10 units with K ending inside the last unit; 272 tiles = one
# whole round of 256 and 16 split in 4 slices of 10; 128 tiles of the
# down projection's width and depth in 2 slices of 60
SPLIT_SHAPES = [(600, 700, 3840), (257, 513, 3088), (4352, 4096, 2560), (4096, 1920, 7680)]


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
@pytest.mark.parametrize("path", ["nvfp4", "int8"])
def test_k_split_tail_tiles(M, N, K, path):
    # the K-split tiles agree with whole tiles to the float32 accumulation
    # bound, and both with the oracle (sampled rows at the large shapes)
    x, w = _case(M, N, K, seed=19)
    wq = Q.nvfp4_encode(w)
    wd = Q.nvfp4_decode(*wq)
    a = Q.nvfp4_encode(x) if path == "nvfp4" else Q.int8_encode(x)
    ys = _run_ws(path, a, wq, M, N, K, split=True)
    yw = _run_ws(path, a, wq, M, N, K, split=False)
    rows = sample_rows(M, 256, seed=5) if M > 1024 else np.arange(M)
    if path == "nvfp4":
        ad = Q.nvfp4_decode(a[0][rows], a[1][rows], a[2])
    else:
        ad = Q.int8_decode(a[0][rows], a[1][rows])
    ref = G.linear_ref(ad, wd)
    bound = _elementwise_bound(ad, wd, K)
    for y in (ys, yw):
        assert np.all(np.abs(y[rows] - ref) <= bound), float(np.max(np.abs(y[rows] - ref) / bound))
    # whole against split over every output (a wrong or missing slice would
    # be off by a whole partial sum, a relative error near 1/slices)
    assert rel_fro(ys, yw) <= 1e-5


def test_k_split_exact_sums_bias_gelu():
    # small integer operands: every partial and every slice sum is exact in
    # float32, so split and whole tiles give the same bits (bias and GELU
    # applied once, by the slice that finishes last)
    # (unit weight scales and power-of-two tensor and row scales: every
    # partial sum is a multiple of 1/2 below 2^23)
    M, N, K = 600, 700, 3840
    rng = np.random.default_rng(23)
    q = rng.integers(-127, 128, (M, K), dtype=np.int8)
    s = np.float32(2.0) ** rng.integers(-4, 4, M).astype(np.float32)
    wq = (rng.integers(0, 256, (N, K // 2), dtype=np.uint8),
          np.full((N, K // 16), 0x38, np.uint8), np.float32(0.125))
    ref = G.linear_ref(Q.int8_decode(q, s), Q.nvfp4_decode(*wq))
    np.testing.assert_array_equal(_run_ws("int8", (q, s), wq, M, N, K, split=True), ref)
    bias = F.f64_to_bf16_rne(rng.normal(0, 0.5, N))
    ys = _run_ws("int8", (q, s), wq, M, N, K, split=True, bias=bias, gelu=True)
    yw = _run_ws("int8", (q, s), wq, M, N, K, split=False, bias=bias, gelu=True)
    np.testing.assert_array_equal(ys, yw)


@pytest.mark.parametrize("path", ["nvfp4", "int8"])
def test_bias_and_gelu(path):
    M, N, K = 200, 300, 256
    x, w = _case(M, N, K, seed=14)
    bias = F.f64_to_bf16_rne(np.random.default_rng(0).standard_normal(N))
    wq = Q.nvfp4_encode(w)
    if path == "nvfp4":
        a = Q.nvfp4_encode(x)
        ref = G.linear_ref(Q.nvfp4_decode(*a), Q.nvfp4_decode(*wq), bias, gelu=True)
        y = run_nvfp4(a, wq, M, N, K, bias=bias, gelu=True)
    else:
        a = Q.int8_encode(x)
        ref = G.linear_ref(Q.int8_decode(*a), Q.nvfp4_decode(*wq), bias, gelu=True)
        y = run_int8(a, wq, M, N, K, bias=bias, gelu=True)
    assert rel_fro(y, _round_ref(ref, False)) <= TOL


@pytest.mark.parametrize("path", ["nvfp4", "int8"])
def test_wide_scale_spread_rows(path):
    # weight rows whose group scales spread over many binades (a group
    # 1e3-1e4 times smaller than the rest of its row)
    M, N, K = 96, 64, 128
    x, w = _case(M, N, K, seed=15)
    wf = F.bf16_to_f64(w)
    wf[3, :16] *= 1e-3
    wf[40, 32:48] *= 1e-4
    w = F.f64_to_bf16_rne(wf)
    wq = Q.nvfp4_encode(w)
    wd = Q.nvfp4_decode(*wq)
    if path == "nvfp4":
        a = Q.nvfp4_encode(x)
        ad = Q.nvfp4_decode(*a)
        run = lambda out_f32: run_nvfp4(a, wq, M, N, K, out_f32=out_f32)
    else:
        a = Q.int8_encode(x)
        ad = Q.int8_decode(*a)
        run = lambda out_f32: run_int8(a, wq, M, N, K, out_f32=out_f32)
    ref = G.linear_ref(ad, wd)
    for out_f32 in (False, True):
        y = run(out_f32)
        assert rel_fro(y, _round_ref(ref, out_f32)) <= TOL
        assert rel_fro(y[:, [3, 40]], _round_ref(ref[:, [3, 40]], out_f32)) <= TOL
    assert np.all(np.abs(y - ref) <= _elementwise_bound(ad, wd, K))


def test_int8_small_integers_exact_f32():
    # unit weight scales, power-of-two tensor and row scales: every partial
    # sum is a multiple of 1/2 below 2^24, exact in float32
    M, N, K = 96, 80, 192
    rng = np.random.default_rng(5)
    q = rng.integers(-127, 128, (M, K), dtype=np.int8)
    s_a = np.float32(2.0) ** rng.integers(-4, 4, M).astype(np.float32)
    w = (rng.integers(0, 256, (N, K // 2), dtype=np.uint8),
         np.full((N, K // 16), 0x38, np.uint8), np.float32(0.125))
    ref = G.linear_ref(Q.int8_decode(q, s_a), Q.nvfp4_decode(*w))
    y = run_int8((q, s_a), w, M, N, K, out_f32=True)
    np.testing.assert_array_equal(y, ref)


def test_power_of_two_scales_exact_f32():
    # all scales powers of two and small K: every partial sum is exact in
    # float32, so the float32 output equals the oracle exactly
    M, N, K = 64, 64, 64
    rng = np.random.default_rng(3)
    a = (rng.integers(0, 256, (M, K // 2), dtype=np.uint8),
         np.full((M, K // 16), 0x38, np.uint8), np.float32(0.5))
    w = (rng.integers(0, 256, (N, K // 2), dtype=np.uint8),
         np.full((N, K // 16), 0x40, np.uint8), np.float32(0.25))
    ref = G.linear_ref(Q.nvfp4_decode(*a), Q.nvfp4_decode(*w))
    y = run_nvfp4(a, w, M, N, K, out_f32=True)
    np.testing.assert_array_equal(y, ref)


@pytest.mark.parametrize("path", ["nvfp4", "int8"])
def test_qkv_full_shape_sampled_rows(path):
    x, w = synth.linear_case(2)
    M, K = x.shape
    N = w.shape[0]
    wq = Q.nvfp4_encode(w)
    wd = Q.nvfp4_decode(*wq)
    rows = sample_rows(M, 192, seed=3)
    if path == "nvfp4":
        a = Q.nvfp4_encode(x)
        y = run_nvfp4(a, wq, M, N, K)
        ref = G.linear_ref(Q.nvfp4_decode(a[0][rows], a[1][rows], a[2]), wd)
    else:
        a = Q.int8_encode(x)
        y = run_int8(a, wq, M, N, K)
        ref = G.linear_ref(Q.int8_decode(a[0][rows], a[1][rows]), wd)
    assert rel_fro(y[rows], _round_ref(ref, False)) <= TOL


@pytest.mark.parametrize("path", ["nvfp4", "int8"])
def test_ffn_full_shape_sampled_rows(path):
    # 1920 -> 7680 (GELU-tanh) -> 1920 on Student-t(3) activations; the
    # down projection's input is the oracle's own hidden activation rows
    x, w_up, w_down = synth.ffn_case(3, M=4096)
    M, K = x.shape
    F_ = w_up.shape[0]
    rows = sample_rows(M, 128, seed=4)
    wu, wdn = Q.nvfp4_encode(w_up), Q.nvfp4_encode(w_down)
    enc = Q.nvfp4_encode if path == "nvfp4" else Q.int8_encode
    run = run_nvfp4 if path == "nvfp4" else run_int8
    dec = (lambda a, r: Q.nvfp4_decode(a[0][r], a[1][r], a[2])) if path == "nvfp4" else \
          (lambda a, r: Q.int8_decode(a[0][r], a[1][r]))
    a = enc(x)
    h = run(a, wu, M, F_, K, gelu=True)
    ref = G.linear_ref(dec(a, rows), Q.nvfp4_decode(*wu), gelu=True)
    assert rel_fro(h[rows], _round_ref(ref, False)) <= TOL
    hb = F.f64_to_bf16_rne(G.linear_ref(dec(a, np.arange(M)), Q.nvfp4_decode(*wu), gelu=True))
    a2 = enc(hb)
    y = run(a2, wdn, M, K, F_)
    ref2 = G.linear_ref(dec(a2, rows), Q.nvfp4_decode(*wdn))
    assert rel_fro(y[rows], _round_ref(ref2, False)) <= TOL


@pytest.mark.parametrize("path", ["nvfp4", "int8"])
@pytest.mark.parametrize("out_f32", [False, True])
def test_strided_output_bias_gelu(path, out_f32):
    # y is a column window of a wider buffer (ldy > N; for bf16 the window
    # starts at a 16-byte boundary, for the second case it does not), with
    # bias and GELU; the columns outside the window must stay untouched
    qa, t = _qa(), torch()
    M, N, K = 300, 200, 192
    x, w = _case(M, N, K, seed=16)
    bias = F.f64_to_bf16_rne(np.random.default_rng(1).standard_normal(N))
    wq = Q.nvfp4_encode(w)
    if path == "nvfp4":
        a = Q.nvfp4_encode(x)
        ref = G.linear_ref(Q.nvfp4_decode(*a), Q.nvfp4_decode(*wq), bias, gelu=True)
    else:
        a = Q.int8_encode(x)
        ref = G.linear_ref(Q.int8_decode(*a), Q.nvfp4_decode(*wq), bias, gelu=True)
    dt = t.float32 if out_f32 else t.bfloat16
    for off in (8, 3):
        ldy = N + 24
        big = t.full((M, ldy), -7.0, dtype=dt, device="cuda")
        y = big[:, off:off + N]
        ws = qa.workspace(qa.qlinear_workspace(qa.NVFP4 if path == "nvfp4" else qa.INT8, M, N, K))
        out = qa.OUT_F32 if out_f32 else qa.OUT_BF16
        if path == "nvfp4":
            qa.qlinear_nvfp4(dev(a[0]), dev(a[1]), dev(np.array([a[2]], np.float32)), dev(wq[0]),
                             dev(wq[1]), dev(np.array([wq[2]], np.float32)), y, M, N, K,
                             bias=dev(bias), out=out, epi=qa.EPI_GELU_TANH, ws=ws, ldy=ldy)
        else:
            qa.qlinear_int8(dev(a[0]), dev(a[1]), dev(wq[0]), dev(wq[1]),
                            dev(np.array([wq[2]], np.float32)), y, M, N, K, bias=dev(bias),
                            out=out, epi=qa.EPI_GELU_TANH, ws=ws, ldy=ldy)
        t.cuda.synchronize()
        got = _out_host(y.contiguous(), out_f32)
        assert rel_fro(got, _round_ref(ref, out_f32)) <= TOL
        rest = t.cat([big[:, :off], big[:, off + N:]], dim=1).float().cpu().numpy()
        assert np.all(rest == -7.0)


def _dev_at_odd_offset(a):
    """Device copy of `a` whose first byte sits at an odd address."""
    raw = np.concatenate([np.zeros(1, np.uint8), np.ascontiguousarray(a).view(np.uint8).ravel()])
    return dev(raw)[1:]


@pytest.mark.parametrize("path", ["nvfp4", "int8"])
@pytest.mark.parametrize("where", ["in_place", "odd_address"])
def test_scale_sources(path, where):
    # K a multiple of 64: the INT8 call reads an aligned weight-scale array
    # in place (it gets no workspace at all); scale arrays at odd addresses
    # go through the per-tile copies in the workspace.  Both must give the
    # oracle's product.
    qa, t = _qa(), torch()
    M, N, K = 300, 200, 192
    x, w = _case(M, N, K, seed=23)
    wq = Q.nvfp4_encode(w)
    put = _dev_at_odd_offset if where == "odd_address" else dev
    y = t.empty((M, N), dtype=t.bfloat16, device="cuda")
    if path == "nvfp4":
        a = Q.nvfp4_encode(x)
        ref = G.linear_ref(Q.nvfp4_decode(*a), Q.nvfp4_decode(*wq))
        ws = qa.workspace(qa.qlinear_workspace(qa.NVFP4, M, N, K))
        qa.qlinear_nvfp4(dev(a[0]), put(a[1]), dev(np.array([a[2]], np.float32)),
                         dev(wq[0]), put(wq[1]), dev(np.array([wq[2]], np.float32)), y, M, N, K,
                         ws=ws)
    else:
        a = Q.int8_encode(x)
        ref = G.linear_ref(Q.int8_decode(*a), Q.nvfp4_decode(*wq))
        ws = None if where == "in_place" else qa.workspace(qa.qlinear_workspace(qa.INT8, M, N, K))
        qa.qlinear_int8(dev(a[0]), dev(a[1]), dev(wq[0]), put(wq[1]),
                        dev(np.array([wq[2]], np.float32)), y, M, N, K, ws=ws)
    t.cuda.synchronize()
    assert rel_fro(_out_host(y, False), _round_ref(ref, False)) <= TOL


QOUT_SHAPES = [(300, 256, 128), (257, 160, 64), (33, 48, 1920), (130, 7680, 1920),
               (300, 256, 3072)]   # the last: K split, its fixup runs the quantizing epilogue


def _qout_case(path, M, N, K, bias, gelu, seed):
    """Operands, oracle output Y (bf16 bits) and the given tensor scale."""
    x, w = _case(M, N, K, seed=seed)
    wq = Q.nvfp4_encode(w)
    a = Q.nvfp4_encode(x) if path == "nvfp4" else Q.int8_encode(x)
    ad = Q.nvfp4_decode(*a) if path == "nvfp4" else Q.int8_decode(*a)
    b = F.f64_to_bf16_rne(np.random.default_rng(seed).standard_normal(N)) if bias else None
    y = F.f64_to_bf16_rne(G.linear_ref(ad, Q.nvfp4_decode(*wq), b, gelu=gelu))
    ts = Q.nvfp4_tensor_scale(y)
    return a, wq, b, y, np.float32(ts)


def _run_qout(path, a, wq, b, ts, M, N, K, gelu, fused):
    """NVFP4 output through the fused epilogue, or through the bf16 output
    and act_quant with the same given tensor scale."""
    qa, t = _qa(), torch()
    fmt = qa.NVFP4 if path == "nvfp4" else qa.INT8
    ws = qa.workspace(qa.qlinear_workspace(fmt, M, N, K))
    epi = qa.EPI_GELU_TANH if gelu else qa.EPI_NONE
    ts_d = dev(np.array([ts], np.float32))
    yq = t.empty((M, N // 2), dtype=t.uint8, device="cuda")
    ys = t.empty((M, N // 16), dtype=t.uint8, device="cuda")
    bias = None if b is None else dev(b)
    wts = dev(np.array([wq[2]], np.float32))
    if fused:
        if path == "nvfp4":
            qa.qlinear_nvfp4_q(dev(a[0]), dev(a[1]), dev(np.array([a[2]], np.float32)), dev(wq[0]),
                               dev(wq[1]), wts, ts_d, yq, ys, M, N, K, bias=bias, epi=epi, ws=ws)
        else:
            qa.qlinear_int8_q(dev(a[0]), dev(a[1]), dev(wq[0]), dev(wq[1]), wts, ts_d, yq, ys, M, N,
                              K, bias=bias, epi=epi, ws=ws)
    else:
        y = t.empty((M, N), dtype=t.bfloat16, device="cuda")
        if path == "nvfp4":
            qa.qlinear_nvfp4(dev(a[0]), dev(a[1]), dev(np.array([a[2]], np.float32)), dev(wq[0]),
                             dev(wq[1]), wts, y, M, N, K, bias=bias, epi=epi, ws=ws)
        else:
            qa.qlinear_int8(dev(a[0]), dev(a[1]), dev(wq[0]), dev(wq[1]), wts, y, M, N, K,
                            bias=bias, epi=epi, ws=ws)
        qa.act_quant(qa.NVFP4, y.view(t.int16), yq, ys, ts_d, qa.TSCALE_GIVEN, None)
    t.cuda.synchronize()
    if not fused:
        _run_qout.last_bf16 = host(y)
    return host(yq), host(ys)


@pytest.mark.parametrize("path", ["nvfp4", "int8"])
@pytest.mark.parametrize("M,N,K", QOUT_SHAPES)
@pytest.mark.parametrize("bias,gelu", [(False, False), (True, True)])
def test_quantized_output(path, M, N, K, bias, gelu):
    # the fused NVFP4 output against the oracle: codes of the oracle's own
    # bf16 output Y, quantized with the same given tensor scale.  The two Y
    # agree to bf16 rounding (the 1e-3 bound above), so a few E2M1 codes sit
    # on the other side of a rounding boundary and move by one code step
    # (up to a third of their group's |max|): at least 99 % of the codes and
    # scales are equal and the decoded outputs agree to 1e-2.  Against the
    # unfused library path (bf16 output, then act_quant with the given
    # scale), which sees the same bf16 values, the bytes are equal.
    a, wq, b, y, ts = _qout_case(path, M, N, K, bias, gelu, seed=17)
    codes, scales = _run_qout(path, a, wq, b, ts, M, N, K, gelu, fused=True)
    oc, os_, _ = Q.nvfp4_encode(y, tscale=ts)
    got = Q.nvfp4_decode(codes, scales, ts)
    ref = Q.nvfp4_decode(oc, os_, ts)
    assert np.mean(codes == oc) >= 0.99 and np.mean(scales == os_) >= 0.99
    assert rel_fro(got, ref) <= 1e-2
    uc, us = _run_qout(path, a, wq, b, ts, M, N, K, gelu, fused=False)
    assert np.array_equal(codes, uc) and np.array_equal(scales, us)
    # and directly: the oracle's NVFP4 encoding (given scale) of the
    # library's own bf16 output equals the fused bytes
    lc, ls, _ = Q.nvfp4_encode(_run_qout.last_bf16, tscale=ts)
    np.testing.assert_array_equal(codes, lc)
    np.testing.assert_array_equal(scales, ls)


def test_quantized_output_saturating_scale():
    # a given tensor scale far below the output's |max|: group scales and
    # codes saturate (E4M3 448, E2M1 6) exactly as act_quant does
    a, wq, b, y, ts = _qout_case("nvfp4", 64, 64, 64, False, False, seed=19)
    small = np.float32(ts / 64)
    codes, scales = _run_qout("nvfp4", a, wq, b, small, 64, 64, 64, False, fused=True)
    uc, us = _run_qout("nvfp4", a, wq, b, small, 64, 64, 64, False, fused=False)
    assert np.array_equal(codes, uc) and np.array_equal(scales, us)
    assert np.any(scales == 0x7E)              # E4M3 448 reached


def _host_amax_bits(y_bits):
    # float bits of max |bf16| over the stored outputs
    return int((np.asarray(y_bits, np.uint16).astype(np.uint32) & 0x7FFF).max()) << 16


# (M, N, K, bias+GELU): ragged rows and columns; bias and GELU; a K-split
# shape (its fixup launch runs the epilogue)
AMAX_SHAPES = [(300, 208, 256, False), (257, 528, 3088, True), (600, 704, 3840, False)]


@pytest.mark.parametrize("M,N,K,bg", AMAX_SHAPES)
@pytest.mark.parametrize("path", ["nvfp4", "int8"])
def test_output_amax_and_amax_given_quant(M, N, K, bg, path):
    # qlinear_*_amax stores the same bf16 output as qlinear_* and the |max|
    # of it; act_quant NVFP4 with that amax given (QA_AMAX_GIVEN) gives the
    # same codes, scales and tensor scale as act_quant's own amax pass
    qa, t = _qa(), torch()
    x, w = _case(M, N, K, seed=29)
    wq = Q.nvfp4_encode(w)
    w3 = (dev(wq[0]), dev(wq[1]), dev(np.array([wq[2]], np.float32)))
    bias = dev(F.f64_to_bf16_rne(np.random.default_rng(3).normal(0, 0.5, N))) if bg else None
    epi = qa.EPI_GELU_TANH if bg else qa.EPI_NONE
    fmt = qa.NVFP4 if path == "nvfp4" else qa.INT8
    ws = qa.workspace(qa.qlinear_workspace(fmt, M, N, K))
    a = Q.nvfp4_encode(x) if path == "nvfp4" else Q.int8_encode(x)
    qws = qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, N))
    qws.zero_()
    amax = qws[:4096].view(t.int32)          # 1024 partial-maximum slots
    y0 = t.empty((M, N), dtype=t.bfloat16, device="cuda")
    y1 = t.empty((M, N), dtype=t.bfloat16, device="cuda")
    if path == "nvfp4":
        a3 = (dev(a[0]), dev(a[1]), dev(np.array([a[2]], np.float32)))
        qa.qlinear_nvfp4(*a3, *w3, y0, M, N, K, bias=bias, epi=epi, ws=ws)
        qa.qlinear_nvfp4_amax(*a3, *w3, y1, amax, M, N, K, bias=bias, epi=epi, ws=ws)
    else:
        a2 = (dev(a[0]), dev(a[1]))
        qa.qlinear_int8(*a2, *w3, y0, M, N, K, bias=bias, epi=epi, ws=ws)
        qa.qlinear_int8_amax(*a2, *w3, y1, amax, M, N, K, bias=bias, epi=epi, ws=ws)
    t.cuda.synchronize()
    yb = host(y1)
    np.testing.assert_array_equal(yb, host(y0))
    assert int(host(amax).astype(np.int64).max()) == _host_amax_bits(yb)
    # the consumer's quantization with the produced amax
    c0, s0, ts0 = qa.empty_nvfp4(M, N)
    c1, s1, ts1 = qa.empty_nvfp4(M, N)
    qa.act_quant(qa.NVFP4, y0.view(t.int16), c0, s0, ts0, 0,
                 qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, N)))
    qa.act_quant(qa.NVFP4, y1.view(t.int16), c1, s1, ts1, qa.AMAX_GIVEN, qws)
    t.cuda.synchronize()
    for u, v in ((c0, c1), (s0, s1), (ts0, ts1)):
        np.testing.assert_array_equal(host(u), host(v))
    # and the oracle's encoding of the same bf16 output
    oc, osc, ots = Q.nvfp4_encode(yb)
    np.testing.assert_array_equal(host(c1), oc)
    np.testing.assert_array_equal(host(s1), osc)
    assert host(ts1)[0] == ots


def test_output_amax_combines_with_preset():
    # the word is max-combined: a larger preset value stays
    qa, t = _qa(), torch()
    M, N, K = 64, 64, 64
    x, w = _case(M, N, K, seed=30)
    a, wq = Q.int8_encode(x), Q.nvfp4_encode(w)
    y = t.empty((M, N), dtype=t.bfloat16, device="cuda")
    big = np.zeros(1024, np.int32)
    big[0] = np.float32(1e30).view(np.int32)
    amax = dev(big)
    qa.qlinear_int8_amax(dev(a[0]), dev(a[1]), dev(wq[0]), dev(wq[1]),
                         dev(np.array([wq[2]], np.float32)), y, amax, M, N, K,
                         ws=qa.workspace(qa.qlinear_workspace(qa.INT8, M, N, K)))
    t.cuda.synchronize()
    got = host(amax)
    assert got[0] == big[0] and got.max() == big[0] and (got[1:] < big[0]).all()
