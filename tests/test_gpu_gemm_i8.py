"""GPU parity of the INT8 linear on integer MFMA (the weight as two int8
digit planes, int8_weight_planes; the linear with w8).

* The int32 sums H and L (qlinear_int8_acc) are bit-exact against the
  oracle's integer form of the weight (oracle.gemm: int8_weight_integers,
  int8_digits, int8_accumulators).
* float32 outputs: y = fl(fl(fl(256 H + L) 2^(X-1)) fl(s_a s_Tw)), three
  roundings of exact values, so |y - Y| <= 4 * 2^-24 |Y| element by element
  against the oracle's exact Y = s_a s_Tw 2^(X-1) (256 H + L) (while |H|,
  |L| < 2^24, which holds for these shapes); bf16 outputs within 1e-3
  relative Frobenius of the float64 oracle rounded to bf16.
* Weights with irregular rows are refused at set-up.
"""
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


def planes(wq, N, K):
    """The weight's digit planes on the device (set-up call)."""
    qa = _qa()
    w8 = qa.empty_int8_planes(N, K)
    assert qa.int8_weight_planes(dev(wq[0]), dev(wq[1]), w8, N, K) == 0
    return w8


def _case(M, N, K, seed, dist="normal"):
    x = synth.activations(seed, M, K, dist, min(4, K // 16), 20.0 if dist == "normal" else 1.0)
    w = synth.weight(seed, 0, N, K)
    return x, w


def run_acc(q, w8, M, N, K, rows=None):
    qa, t = _qa(), torch()
    hi = t.empty((M, N), dtype=t.int32, device="cuda")
    lo = t.empty((M, N), dtype=t.int32, device="cuda")
    qa.qlinear_int8_acc(dev(q), w8, hi, lo, M, N, K)
    t.cuda.synchronize()
    if rows is not None:
        idx = t.from_numpy(rows).cuda()
        hi, lo = hi.index_select(0, idx), lo.index_select(0, idx)
    return host(hi).astype(np.int64), host(lo).astype(np.int64)


def run_i8(a, wq, w8, M, N, K, bias=None, out_f32=False, gelu=False, ws=True, ldy=None,
           y=None):
    qa, t = _qa(), torch()
    if y is None:
        y = t.empty((M, N), dtype=t.float32 if out_f32 else t.bfloat16, device="cuda")
    wsb = qa.workspace(qa.qlinear_workspace(qa.INT8, M, N, K)) if ws else None
    qa.qlinear_int8(dev(a[0]), dev(a[1]), None, None, dev(np.array([wq[2]], np.float32)), y, M,
                    N, K, bias=None if bias is None else dev(bias),
                    out=qa.OUT_F32 if out_f32 else qa.OUT_BF16,
                    epi=qa.EPI_GELU_TANH if gelu else qa.EPI_NONE, ws=wsb, ldy=ldy, w8=w8)
    t.cuda.synchronize()
    return y


def _out(y, out_f32):
    return host(y).astype(np.float64) if out_f32 else F.bf16_to_f64(host(y))


def _oracle_sums(q, wq, rows=None):
    integer, X, regular = G.int8_weight_integers(wq[0], wq[1])
    assert regular.all()
    hi, lo = G.int8_digits(integer)
    qq = q if rows is None else q[rows]
    H, L = G.int8_accumulators(qq, hi, lo)
    return H, L, X


# ragged M, N and K (K = 48: one unit that K ends inside; 80, 176: an odd
# number of units), a single row, N not a multiple of 4
SHAPES = [(256, 256, 256), (1, 16, 16), (300, 200, 48), (257, 300, 80), (77, 90, 112),
          (513, 257, 96), (130, 129, 176), (64, 5760, 1920), (70, 1920, 7680)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_int32_sums_bit_exact(M, N, K):
    x, w = _case(M, N, K, seed=41)
    q, _ = Q.int8_encode(x)
    wq = Q.nvfp4_encode(w)
    H, L, _ = _oracle_sums(q, wq)
    gh, gl = run_acc(q, planes(wq, N, K), M, N, K)
    np.testing.assert_array_equal(gh, H)
    np.testing.assert_array_equal(gl, L)


def test_int32_sums_bit_exact_full_qkv_shape():
    # the QKV configuration (17776 x 1920 -> 5760) on sampled rows, the
    # ragged last tile included
    x, w = synth.linear_case(2)
    M, K = x.shape
    N = w.shape[0]
    q, _ = Q.int8_encode(x)
    wq = Q.nvfp4_encode(w)
    rows = sample_rows(M, 160, seed=6)
    H, L, _ = _oracle_sums(q, wq, rows)
    gh, gl = run_acc(q, planes(wq, N, K), M, N, K, rows=rows)
    np.testing.assert_array_equal(gh, H)
    np.testing.assert_array_equal(gl, L)


def test_int32_sums_extreme_digits():
    # every activation +-127 and weights whose rows span exactly 7 octaves
    # (the largest digits: |hi| up to 90, lo at -128 and 127)
    rng = np.random.default_rng(43)
    M, N, K = 96, 64, 512
    q = np.where(rng.random((M, K)) < 0.5, -127, 127).astype(np.int8)
    codes = rng.integers(0, 16, (N, K // 2), dtype=np.uint8)
    scales = np.where(rng.random((N, K // 16)) < 0.5, 0x77, 0x3E).astype(np.uint8)
    scales[:, 0], scales[:, 1] = 0x77, 0x3E            # 15*2^4 and 14*2^-3: span 7
    wq = (codes, scales, np.float32(1.0))
    integer, _, regular = G.int8_weight_integers(codes, scales)
    assert regular.all()
    hi, lo = G.int8_digits(integer)
    assert np.abs(hi.astype(int)).max() == 90 and lo.min() <= -64
    H, L, _ = _oracle_sums(q, wq)
    gh, gl = run_acc(q, planes(wq, N, K), M, N, K)
    np.testing.assert_array_equal(gh, H)
    np.testing.assert_array_equal(gl, L)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_f32_output_elementwise(M, N, K):
    x, w = _case(M, N, K, seed=42)
    a = Q.int8_encode(x)
    wq = Q.nvfp4_encode(w)
    H, L, X = _oracle_sums(a[0], wq)
    Y = G.int8_linear_from_sums(H, L, X, a[1], wq[2])
    y = _out(run_i8(a, wq, planes(wq, N, K), M, N, K, out_f32=True), True)
    assert np.all(np.abs(y - Y) <= 4 * 2.0 ** -24 * np.abs(Y)), float(np.max(np.abs(y - Y)))
    # and the dequantized float64 product (the layer's definition)
    ref = G.linear_ref(Q.int8_decode(*a), Q.nvfp4_decode(*wq))
    assert rel_fro(y, ref.astype(np.float32)) <= 1e-6


@pytest.mark.parametrize("M,N,K", SHAPES[:6])
@pytest.mark.parametrize("bias,gelu", [(False, False), (True, False), (False, True), (True, True)])
def test_bf16_output(M, N, K, bias, gelu):
    x, w = _case(M, N, K, seed=44)
    a = Q.int8_encode(x)
    wq = Q.nvfp4_encode(w)
    b = F.f64_to_bf16_rne(np.random.default_rng(2).normal(0, 0.5, N)) if bias else None
    ref = G.linear_ref(Q.int8_decode(*a), Q.nvfp4_decode(*wq), b, gelu=gelu)
    y = _out(run_i8(a, wq, planes(wq, N, K), M, N, K, bias=b, gelu=gelu), False)
    assert rel_fro(y, F.bf16_to_f64(F.f64_to_bf16_rne(ref))) <= TOL


def test_zero_activation_rows():
    # an all-zero token row quantizes to q = 0, s = 0 (INT8 reading): its
    # output is exactly the bias (or 0), on both INT8 kernels
    qa = _qa()
    M, N, K = 130, 96, 256
    x, w = _case(M, N, K, seed=45)
    x[[0, 57, 129]] = 0
    a = Q.int8_encode(x)
    assert a[1][0] == 0 and not a[0][57].any()
    wq = Q.nvfp4_encode(w)
    b = F.f64_to_bf16_rne(np.random.default_rng(5).normal(0, 1, N))
    w8 = planes(wq, N, K)
    t = torch()
    for use_w8 in (True, False):
        y = t.empty((M, N), dtype=t.float32, device="cuda")
        qa.qlinear_int8(dev(a[0]), dev(a[1]), dev(wq[0]), dev(wq[1]),
                        dev(np.array([wq[2]], np.float32)), y, M, N, K, bias=dev(b),
                        out=qa.OUT_F32, ws=qa.workspace(qa.qlinear_workspace(qa.INT8, M, N, K)),
                        w8=w8 if use_w8 else None)
        t.cuda.synchronize()
        got = host(y).astype(np.float64)
        for r in (0, 57, 129):
            np.testing.assert_array_equal(got[r], F.bf16_to_f64(b))
        ref = G.linear_ref(Q.int8_decode(*a), Q.nvfp4_decode(*wq), b)
        assert rel_fro(got, ref) <= 1e-6


# shapes whose last round of 256 x 128 tiles is split along K: 3 x 6 = 18
# tiles in 4 slices of 15 units; 70 x 15 = 1050 = 4 x 256 + 26 (the 2B
# down projection) in 4 slices of 30
SPLIT_SHAPES = [(600, 700, 3840), (17776, 1920, 7680)]


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
def test_k_split_identical_to_whole_tiles(M, N, K):
    # integer partial sums: the split and the unsplit call give the same bits
    qa = _qa()
    x, w = _case(M, N, K, seed=46)
    a = Q.int8_encode(x)
    wq = Q.nvfp4_encode(w)
    w8 = planes(wq, N, K)
    full = qa.qlinear_workspace(qa.INT8, M, N, K)
    assert full > 0
    t = torch()
    ys = run_i8(a, wq, w8, M, N, K, out_f32=True)
    yw = run_i8(a, wq, w8, M, N, K, out_f32=True, ws=False)
    np.testing.assert_array_equal(host(ys), host(yw))
    rows = sample_rows(M, 96, seed=7)
    H, L, X = _oracle_sums(a[0], wq, rows)
    Y = G.int8_linear_from_sums(H, L, X, a[1][rows], wq[2])
    got = host(ys).astype(np.float64)[rows]
    assert np.all(np.abs(got - Y) <= 4 * 2.0 ** -24 * np.abs(Y))


def test_strided_output_window():
    # y a column window of a wider buffer (16-byte aligned and not): the
    # columns outside stay untouched
    qa, t = _qa(), torch()
    M, N, K = 300, 200, 192
    x, w = _case(M, N, K, seed=47)
    a = Q.int8_encode(x)
    wq = Q.nvfp4_encode(w)
    w8 = planes(wq, N, K)
    b = F.f64_to_bf16_rne(np.random.default_rng(1).standard_normal(N))
    ref = G.linear_ref(Q.int8_decode(*a), Q.nvfp4_decode(*wq), b, gelu=True)
    for out_f32 in (False, True):
        dt = t.float32 if out_f32 else t.bfloat16
        for off in (8, 3):
            ldy = N + 24
            big = t.full((M, ldy), -7.0, dtype=dt, device="cuda")
            y = big[:, off:off + N]
            run_i8(a, wq, w8, M, N, K, bias=b, gelu=True, out_f32=out_f32, ldy=ldy, y=y)
            got = _out(y.contiguous(), out_f32)
            want = ref.astype(np.float32).astype(np.float64) if out_f32 else \
                F.bf16_to_f64(F.f64_to_bf16_rne(ref))
            assert rel_fro(got, want) <= TOL
            rest = t.cat([big[:, :off], big[:, off + N:]], dim=1).float().cpu().numpy()
            assert np.all(rest == -7.0)


@pytest.mark.parametrize("M,N,K", [(300, 256, 128), (33, 48, 1920), (600, 704, 3840)])
def test_quantized_output_and_amax(M, N, K):
    # the fused NVFP4 output and the output |max| of the integer kernel: the
    # bytes equal act_quant of its own bf16 output (given scale), and the
    # |max| equals the host maximum of that output
    qa, t = _qa(), torch()
    x, w = _case(M, N, K, seed=48)
    a = Q.int8_encode(x)
    wq = Q.nvfp4_encode(w)
    w8 = planes(wq, N, K)
    wts = dev(np.array([wq[2]], np.float32))
    ws = qa.workspace(qa.qlinear_workspace(qa.INT8, M, N, K))
    y = t.empty((M, N), dtype=t.bfloat16, device="cuda")
    slots = qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, N))
    slots.zero_()
    amax = slots[:4096].view(t.int32)
    qa.qlinear_int8_amax(dev(a[0]), dev(a[1]), None, None, wts, y, amax, M, N, K, ws=ws, w8=w8)
    t.cuda.synchronize()
    yb = host(y)
    assert int(host(amax).astype(np.int64).max()) == \
        int((yb.astype(np.uint32) & 0x7FFF).max()) << 16
    ts = np.float32(Q.nvfp4_tensor_scale(yb))
    ts_d = dev(np.array([ts], np.float32))
    yq = t.empty((M, N // 2), dtype=t.uint8, device="cuda")
    ys = t.empty((M, N // 16), dtype=t.uint8, device="cuda")
    qa.qlinear_int8_q(dev(a[0]), dev(a[1]), None, None, wts, ts_d, yq, ys, M, N, K, ws=ws, w8=w8)
    t.cuda.synchronize()
    oc, osc, _ = Q.nvfp4_encode(yb, tscale=ts)
    np.testing.assert_array_equal(host(yq), oc)
    np.testing.assert_array_equal(host(ys), osc)


# shapes that run the persistent whole-tile kernel (more than 256 whole
# tiles, an even number of 6 .. 64 units), all with ragged M: 288 tiles (32
# workgroups take a second tile) with ragged N at 30 and 6 units; 432 tiles
# at 64 units; 540 tiles whose last round is split along K (512 whole
# tiles, two per workgroup, then the slices and their fixup)
PERSIST_SHAPES = [(4452, 1960, 1920), (4452, 1960, 384), (4452, 2984, 4096), (4452, 3840, 3840)]


@pytest.mark.parametrize("M,N,K", PERSIST_SHAPES)
def test_persistent_tiles(M, N, K):
    qa, t = _qa(), torch()
    x, w = _case(M, N, K, seed=51)
    a = Q.int8_encode(x)
    wq = Q.nvfp4_encode(w)
    w8 = planes(wq, N, K)
    rows = sample_rows(M, 24, seed=52)
    # float32 outputs element by element on sampled rows (every tile row's
    # first rows, the ragged last tile row, all columns)
    rows = np.union1d(rows, np.arange(0, M, 256))
    H, L, X = _oracle_sums(a[0], wq, rows)
    Y = G.int8_linear_from_sums(H, L, X, a[1][rows], wq[2])
    y = _out(run_i8(a, wq, w8, M, N, K, out_f32=True), True)[rows]
    assert np.all(np.abs(y - Y) <= 4 * 2.0 ** -24 * np.abs(Y)), float(np.max(np.abs(y - Y)))
    # bf16 with bias and GELU (the staged epilogue, ragged columns in the
    # last tile column)
    b = F.f64_to_bf16_rne(np.random.default_rng(3).normal(0, 0.5, N))
    ref = G.linear_ref(Q.int8_decode(a[0][rows], a[1][rows]), Q.nvfp4_decode(*wq), b, gelu=True)
    yb = _out(run_i8(a, wq, w8, M, N, K, bias=b, gelu=True), False)[rows]
    assert rel_fro(yb, F.bf16_to_f64(F.f64_to_bf16_rne(ref))) <= TOL
    # plain bf16 output with its |max|, then the NVFP4 output: the codes
    # equal act_quant of the kernel's own bf16 output (given scale)
    wts = dev(np.array([wq[2]], np.float32))
    ws = qa.workspace(qa.qlinear_workspace(qa.INT8, M, N, K))
    yy = t.empty((M, N), dtype=t.bfloat16, device="cuda")
    slots = qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, N))
    slots.zero_()
    amax = slots[:4096].view(t.int32)
    qa.qlinear_int8_amax(dev(a[0]), dev(a[1]), None, None, wts, yy, amax, M, N, K, ws=ws, w8=w8)
    t.cuda.synchronize()
    yh = host(yy)
    assert int(host(amax).astype(np.int64).max()) == \
        int((yh.astype(np.uint32) & 0x7FFF).max()) << 16
    if N % 16 == 0:
        ts = np.float32(Q.nvfp4_tensor_scale(yh))
        yq = t.empty((M, N // 2), dtype=t.uint8, device="cuda")
        ys = t.empty((M, N // 16), dtype=t.uint8, device="cuda")
        qa.qlinear_int8_q(dev(a[0]), dev(a[1]), None, None, wts, dev(np.array([ts], np.float32)),
                          yq, ys, M, N, K, ws=ws, w8=w8)
        t.cuda.synchronize()
        oc, osc, _ = Q.nvfp4_encode(yh[rows], tscale=ts)
        np.testing.assert_array_equal(host(yq)[rows], oc)
        np.testing.assert_array_equal(host(ys)[rows], osc)


def test_irregular_rows_refused():
    # rows whose non-zero group scales span 8 or more octaves have no
    # two-digit form: the set-up call counts them and refuses
    qa = _qa()
    N, K = 40, 64
    rng = np.random.default_rng(49)
    codes = rng.integers(0, 16, (N, K // 2), dtype=np.uint8)
    scales = np.full((N, K // 16), 0x50, np.uint8)
    scales[[3, 17, 39], 0] = 0x7E
    scales[[3, 17, 39], 1] = 0x30        # 14 * 2^5 against 8 * 2^-4: span 9
    _, _, regular = G.int8_weight_integers(codes, scales)
    assert (~regular).sum() == 3
    w8 = qa.empty_int8_planes(N, K)
    st, n_irr = qa.int8_weight_planes_count(dev(codes), dev(scales), w8, N, K)
    assert st == -4 and n_irr == 3
    # the layer still runs exactly without the planes (fp16 kernel)
    q = rng.integers(-127, 128, (8, K), dtype=np.int8)
    s = np.ones(8, np.float32)
    t = torch()
    y = t.empty((8, N), dtype=t.float32, device="cuda")
    qa.qlinear_int8(dev(q), dev(s), dev(codes), dev(scales), dev(np.ones(1, np.float32)), y, 8, N,
                    K, out=qa.OUT_F32, ws=qa.workspace(qa.qlinear_workspace(qa.INT8, 8, N, K)))
    t.cuda.synchronize()
    ref = G.linear_ref(q.astype(np.float64), Q.nvfp4_decode(codes, scales, np.float32(1)))
    assert rel_fro(host(y), ref) <= 1e-6


def test_layer_call_with_planes():
    # qlinear (act_quant + the linear) with w8 equals act_quant then
    # qlinear_int8 with w8, bit for bit
    qa, t = _qa(), torch()
    M, N, K = 300, 256, 384
    x, w = _case(M, N, K, seed=50)
    wq = Q.nvfp4_encode(w)
    w8 = planes(wq, N, K)
    wts = dev(np.array([wq[2]], np.float32))
    xd = dev(x).view(t.int16)
    y1 = t.empty((M, N), dtype=t.bfloat16, device="cuda")
    qa.qlinear(qa.INT8, xd, None, None, None, wts, y1, M, N, K,
               ws=qa.workspace(qa.qlinear_layer_workspace(qa.INT8, M, N, K)), w8=w8)
    a = Q.int8_encode(x)
    y2 = run_i8(a, wq, w8, M, N, K)
    t.cuda.synchronize()
    np.testing.assert_array_equal(host(y1), host(y2))
