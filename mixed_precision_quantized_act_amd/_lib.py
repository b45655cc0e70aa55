"""ctypes binding of libqact.so (the C ABI declared in include/qact.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every computation runs in the library's HIP kernels.
There is no fallback: if the library is missing, loading fails loudly.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqact.so")

NVFP4, INT8 = 0, 1
OUT_BF16, OUT_F32 = 0, 1
EPI_NONE, EPI_GELU_TANH = 0, 1
TSCALE_GIVEN = 1
AMAX_GIVEN = 2
NOALLOC_SCRATCH_BYTES = 64 << 20     # QA_NOALLOC_SCRATCH_BYTES


class QactError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_SIGS = {
    "qa_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "qa_build_info": (ctypes.c_char_p, []),
    "act_quant_workspace": (_SZ, [ctypes.c_int, _I64, _I64]),
    "act_quant": (ctypes.c_int, [ctypes.c_int, _P, _I64, _I64, _I64, _P, _P, _P, ctypes.c_uint32,
                                 _P, _SZ, _P]),
    "qlinear_workspace": (_SZ, [ctypes.c_int, _I64, _I64, _I64]),
    "qlinear_nvfp4": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _I64,
                                     ctypes.c_int, ctypes.c_int, _P, _SZ, _P]),
    "qlinear_int8": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _I64,
                                    ctypes.c_int, ctypes.c_int, _P, _SZ, _P]),
    "qlinear_int8_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P,
                                            _I64, ctypes.c_int, ctypes.c_int, _P]),
    "int8_weight_planes_bytes": (_SZ, [_I64, _I64]),
    "int8_weight_planes": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _SZ, _P, _P]),
    "qlinear_int8_acc": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, _P, _P, _P]),
    "qlinear_nvfp4_q": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_int,
                                       _P, _P, _P, _P, _SZ, _P]),
    "qlinear_int8_q": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_int,
                                      _P, _P, _P, _P, _SZ, _P]),
    "qlinear_nvfp4_amax": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _I64,
                                          ctypes.c_int, _P, _P, _SZ, _P]),
    "qlinear_int8_amax": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _I64,
                                         ctypes.c_int, _P, _P, _SZ, _P]),
    "qlinear_layer_workspace": (_SZ, [ctypes.c_int, _I64, _I64, _I64]),
    "qlinear": (ctypes.c_int, [ctypes.c_int, _P, _I64, _P, ctypes.c_uint32, _P, _P, _P, _P, _I64,
                               _I64, _I64, _P, _P, _I64, ctypes.c_int, ctypes.c_int, _P, _SZ, _P]),
    "act_quant_routed": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, _P, _P, _P, ctypes.c_uint32, _P,
                                        _SZ, _P, _P, _P]),
    "qlinear_routed_workspace": (_SZ, [_I64, _I64, _I64]),
    "qlinear_routed": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64,
                                      _P, _P, _I64, ctypes.c_int, _P, _P, _SZ, _P]),
    "tdc_update_ring": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _P, _P, _SZ, _P]),
    "tdc_apply_ring": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _P, _P, _P, _SZ, _P]),
    "reduce_workspace": (_SZ, [_I64]),
    "block_gamma": (ctypes.c_int, [_P, _P, _I64, _P, _P, _SZ, _P]),
    "tdc_update": (ctypes.c_int, [_P, _P, _P, _P, _I64, _P, _P, _SZ, _P]),
    "tdc_apply": (ctypes.c_int, [_P, _P, _P, _I64, _P, _P, _SZ, _P]),
    "tdc_apply_amax": (ctypes.c_int, [_P, _P, _P, _I64, _P, _P, _P, _SZ, _P]),
    "rel_err": (ctypes.c_int, [_P, _P, _I64, _P, _P, _SZ, _P]),
    "delta_cosine": (ctypes.c_int, [_P, _P, _I64, _P, _P, _SZ, _P]),
    "tdc_decide_cos": (ctypes.c_int, [ctypes.c_int, _P, _P, ctypes.c_int, ctypes.c_double, _P]),
    "qa_cosine_from_sums": (ctypes.c_double, [_P]),
    "dmpq_fit": (ctypes.c_int, [_P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P, _P]),
    "dmpq_mask": (ctypes.c_int, [_P, ctypes.c_int, ctypes.c_int, _P, _P, ctypes.c_double, _P]),
    "tdc_decide": (ctypes.c_int, [ctypes.c_int, _P, _P, ctypes.c_int, ctypes.c_double, _P]),
    "qa_set_gemm_events": (ctypes.c_int, [_P, _P]),
    "qa_test_convert": (ctypes.c_int, [ctypes.c_int, ctypes.c_uint32, _I64, _P, _P]),
    "qa_test_stage_ab": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, _P, _P, _P]),
    "qa_set_gate": (ctypes.c_int, [_P, ctypes.c_uint32]),
    "qa_decide_step": (ctypes.c_int, [_P, _P, _P, ctypes.c_double, ctypes.c_double, ctypes.c_int,
                                      ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _P]),
    "qa_gamma_from_sums": (ctypes.c_double, [_P]),
    "qa_rel_l2_from_sums": (ctypes.c_double, [_P]),
    "qa_rel_err_from_sums": (ctypes.c_double, [_P]),
}

EXPORTS = tuple(_SIGS)


def lib():
    """The loaded library (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libqact.so is not built at {LIB_PATH}; run "
                              "python -m mixed_precision_quantized_act_amd.build")
        # torch first: its HIP runtime (listed by torch's libraries as
        # libamdhip64.so) then provides the libamdhip64.so.7 the library
        # needs.  Loaded the other way round, the process holds two HIP
        # runtimes, and whichever touches the GPU second finds no device.
        import torch  # noqa: F401
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype, f.argtypes = res, args
        _lib = h
    return _lib


def _check(fn, status):
    if status != 0:
        raise QactError(fn, status, lib().qa_strerror(status).decode())


def _ptr(t):
    # ctypes converts a plain int for a c_void_p parameter
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def strerror(status):
    return lib().qa_strerror(status).decode()


def build_info():
    return lib().qa_build_info().decode()


# --------------------------------------------------------------- act_quant --

def act_quant_workspace(fmt, M, K):
    return lib().act_quant_workspace(fmt, M, K)


def act_quant(fmt, x, q, scales, tscale=None, flags=0, ws=None, M=None, K=None, ldx=None,
              stream=None):
    """Quantize bf16 x [M, ldx] (first K columns) into q / scales (/ tscale)."""
    M = x.shape[0] if M is None else M
    K = x.shape[1] if K is None else K
    ldx = x.stride(0) if ldx is None else ldx
    _check("act_quant", lib().act_quant(fmt, _ptr(x), M, K, ldx, _ptr(q), _ptr(scales),
                                        _ptr(tscale), flags, _ptr(ws), _nbytes(ws),
                                        _stream(stream)))


# ----------------------------------------------------------------- qlinear --

def qlinear_workspace(fmt, M, N, K):
    return lib().qlinear_workspace(fmt, M, N, K)


def qlinear_nvfp4(a_q, a_s, a_ts, w_q, w_s, w_ts, y, M, N, K, bias=None, out=OUT_BF16,
                  epi=EPI_NONE, ws=None, ldy=None, stream=None):
    ldy = y.stride(0) if ldy is None else ldy
    _check("qlinear_nvfp4", lib().qlinear_nvfp4(
        _ptr(a_q), _ptr(a_s), _ptr(a_ts), _ptr(w_q), _ptr(w_s), _ptr(w_ts), M, N, K, _ptr(bias),
        _ptr(y), ldy, out, epi, _ptr(ws), _nbytes(ws), _stream(stream)))


def qlinear_int8(a_q, a_s, w_q, w_s, w_ts, y, M, N, K, bias=None, out=OUT_BF16, epi=EPI_NONE,
                 ws=None, ldy=None, stream=None, w8=None):
    """INT8 linear; w8 (the weight's digit planes) selects the integer-MFMA kernel."""
    ldy = y.stride(0) if ldy is None else ldy
    _check("qlinear_int8", lib().qlinear_int8(
        _ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s), _ptr(w_ts), _ptr(w8), M, N, K, _ptr(bias),
        _ptr(y), ldy, out, epi, _ptr(ws), _nbytes(ws), _stream(stream)))


def qlinear_int8_noalloc(a_q, a_s, w_q, w_s, w_ts, y, M, N, K, bias=None, out=OUT_BF16,
                         epi=EPI_NONE, ldy=None, stream=None, w8=None):
    """qlinear_int8 with its workspace in the library's static device array
    (NOALLOC_SCRATCH_BYTES per GPU); calls that overlap on one GPU race."""
    ldy = y.stride(0) if ldy is None else ldy
    _check("qlinear_int8_noalloc", lib().qlinear_int8_noalloc(
        _ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s), _ptr(w_ts), _ptr(w8), M, N, K, _ptr(bias),
        _ptr(y), ldy, out, epi, _stream(stream)))


def int8_weight_planes_bytes(N, K):
    return lib().int8_weight_planes_bytes(N, K)


def int8_weight_planes(w_q, w_s, w8, N, K, stream=None):
    """Write the NVFP4 weight's int8 digit planes into w8 (device, set-up;
    synchronises the stream).  Returns the number of irregular rows (0 on
    success); raises QactError (QA_EUNSUPPORTED) when some row is irregular."""
    import ctypes as _c
    cnt = _c.c_int64(0)
    st = lib().int8_weight_planes(_ptr(w_q), _ptr(w_s), N, K, _ptr(w8), _nbytes(w8),
                                  _c.addressof(cnt), _stream(stream))
    _check("int8_weight_planes", st)
    return cnt.value


def int8_weight_planes_count(w_q, w_s, w8, N, K, stream=None):
    """As int8_weight_planes, but returns (status, irregular rows) instead of raising."""
    import ctypes as _c
    cnt = _c.c_int64(0)
    st = lib().int8_weight_planes(_ptr(w_q), _ptr(w_s), N, K, _ptr(w8), _nbytes(w8),
                                  _c.addressof(cnt), _stream(stream))
    return st, cnt.value


def qlinear_int8_acc(a_q, w8, acc_hi, acc_lo, M, N, K, stream=None):
    """The INT8 linear's exact int32 sums H (hi plane) and L (lo plane), [M, N] each."""
    _check("qlinear_int8_acc", lib().qlinear_int8_acc(
        _ptr(a_q), _ptr(w8), M, N, K, _ptr(acc_hi), _ptr(acc_lo), _stream(stream)))


def qlinear_nvfp4_q(a_q, a_s, a_ts, w_q, w_s, w_ts, y_ts, y_q, y_s, M, N, K, bias=None,
                    epi=EPI_NONE, ws=None, stream=None):
    """NVFP4 linear with the output quantized to NVFP4 (given tensor scale y_ts)."""
    _check("qlinear_nvfp4_q", lib().qlinear_nvfp4_q(
        _ptr(a_q), _ptr(a_s), _ptr(a_ts), _ptr(w_q), _ptr(w_s), _ptr(w_ts), M, N, K, _ptr(bias),
        epi, _ptr(y_ts), _ptr(y_q), _ptr(y_s), _ptr(ws), _nbytes(ws), _stream(stream)))


def qlinear_int8_q(a_q, a_s, w_q, w_s, w_ts, y_ts, y_q, y_s, M, N, K, bias=None, epi=EPI_NONE,
                   ws=None, stream=None, w8=None):
    """INT8 linear with the output quantized to NVFP4 (given tensor scale y_ts)."""
    _check("qlinear_int8_q", lib().qlinear_int8_q(
        _ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s), _ptr(w_ts), _ptr(w8), M, N, K, _ptr(bias),
        epi, _ptr(y_ts), _ptr(y_q), _ptr(y_s), _ptr(ws), _nbytes(ws), _stream(stream)))


def qlinear_nvfp4_amax(a_q, a_s, a_ts, w_q, w_s, w_ts, y, y_amax, M, N, K, bias=None,
                       epi=EPI_NONE, ws=None, ldy=None, stream=None):
    """qlinear_nvfp4 (bf16 out) that also max-combines |y| into y_amax."""
    ldy = y.stride(0) if ldy is None else ldy
    _check("qlinear_nvfp4_amax", lib().qlinear_nvfp4_amax(
        _ptr(a_q), _ptr(a_s), _ptr(a_ts), _ptr(w_q), _ptr(w_s), _ptr(w_ts), M, N, K, _ptr(bias),
        _ptr(y), ldy, epi, _ptr(y_amax), _ptr(ws), _nbytes(ws), _stream(stream)))


def qlinear_int8_amax(a_q, a_s, w_q, w_s, w_ts, y, y_amax, M, N, K, bias=None, epi=EPI_NONE,
                      ws=None, ldy=None, stream=None, w8=None):
    """qlinear_int8 (bf16 out) that also max-combines |y| into y_amax."""
    ldy = y.stride(0) if ldy is None else ldy
    _check("qlinear_int8_amax", lib().qlinear_int8_amax(
        _ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s), _ptr(w_ts), _ptr(w8), M, N, K, _ptr(bias),
        _ptr(y), ldy, epi, _ptr(y_amax), _ptr(ws), _nbytes(ws), _stream(stream)))


def qlinear_layer_workspace(fmt, M, N, K):
    return lib().qlinear_layer_workspace(fmt, M, N, K)


def qlinear(fmt, x, x_ts, w_q, w_s, w_ts, y, M, N, K, bias=None, out=OUT_BF16, epi=EPI_NONE,
            flags=0, ws=None, ldx=None, ldy=None, stream=None, w8=None):
    ldx = x.stride(0) if ldx is None else ldx
    ldy = y.stride(0) if ldy is None else ldy
    _check("qlinear", lib().qlinear(
        fmt, _ptr(x), ldx, _ptr(x_ts), flags, _ptr(w_q), _ptr(w_s), _ptr(w_ts), _ptr(w8), M, N,
        K, _ptr(bias), _ptr(y), ldy, out, epi, _ptr(ws), _nbytes(ws), _stream(stream)))


# ------------------------------------------------------------- Gamma / TDC --

def act_quant_routed(route, x, q4, s4, ts4, flags4, ws4, q8, s8, M=None, K=None, ldx=None,
                     stream=None):
    """act_quant in the format the device byte route[0] selects (1 NVFP4,
    2 INT8, 0 nothing), one launch."""
    M = x.shape[0] if M is None else M
    K = x.shape[1] if K is None else K
    ldx = x.stride(0) if ldx is None else ldx
    _check("act_quant_routed", lib().act_quant_routed(
        _ptr(route), _ptr(x), M, K, ldx, _ptr(q4), _ptr(s4), _ptr(ts4), flags4, _ptr(ws4),
        _nbytes(ws4), _ptr(q8), _ptr(s8), _stream(stream)))


def qlinear_routed_workspace(M, N, K):
    return lib().qlinear_routed_workspace(M, N, K)


def qlinear_routed(route, a_q4, a_s4, a_ts4, a_q8, a_s8, w_q, w_s, w_ts, w8, y, M, N, K,
                   bias=None, epi=EPI_NONE, y_amax=None, ws=None, ldy=None, stream=None):
    """The linear in the format the device byte route[0] selects (1 NVFP4
    on (a_q4, a_s4, a_ts4), 2 INT8 on (a_q8, a_s8) with w8, 0 nothing):
    one GEMM launch for both formats; bf16 y, y_amax as for *_amax."""
    ldy = y.stride(0) if ldy is None else ldy
    _check("qlinear_routed", lib().qlinear_routed(
        _ptr(route), _ptr(a_q4), _ptr(a_s4), _ptr(a_ts4), _ptr(a_q8), _ptr(a_s8), _ptr(w_q),
        _ptr(w_s), _ptr(w_ts), _ptr(w8), M, N, K, _ptr(bias), _ptr(y), ldy, epi, _ptr(y_amax),
        _ptr(ws), _nbytes(ws), _stream(stream)))


def tdc_update_ring(blk, x_in, x_out, ring0, ring1, sums4, ws, n=None, stream=None):
    """tdc_update with the ring slot from the device byte blk[0]."""
    n = x_in.numel() if n is None else n
    _check("tdc_update_ring", lib().tdc_update_ring(
        _ptr(blk), _ptr(x_in), _ptr(x_out), _ptr(ring0), _ptr(ring1), n, _ptr(sums4), _ptr(ws),
        _nbytes(ws), _stream(stream)))


def tdc_apply_ring(blk, x_in, ring0, ring1, x_out, sums2=None, ws=None, out_amax=None, n=None,
                   stream=None):
    """tdc_apply (and tdc_apply_amax with out_amax) of the ring slot that
    the device byte blk[0] selects."""
    n = x_in.numel() if n is None else n
    _check("tdc_apply_ring", lib().tdc_apply_ring(
        _ptr(blk), _ptr(x_in), _ptr(ring0), _ptr(ring1), _ptr(x_out), n, _ptr(sums2),
        _ptr(out_amax), _ptr(ws), _nbytes(ws), _stream(stream)))


def reduce_workspace(n):
    return lib().reduce_workspace(n)


def block_gamma(x_in, x_out, sums2, ws, n=None, stream=None):
    n = x_in.numel() if n is None else n
    _check("block_gamma", lib().block_gamma(_ptr(x_in), _ptr(x_out), n, _ptr(sums2), _ptr(ws),
                                            _nbytes(ws), _stream(stream)))


def tdc_update(x_in, x_out, delta_prev, delta_new, sums4, ws, n=None, stream=None):
    n = x_in.numel() if n is None else n
    _check("tdc_update", lib().tdc_update(_ptr(x_in), _ptr(x_out), _ptr(delta_prev),
                                          _ptr(delta_new), n, _ptr(sums4), _ptr(ws), _nbytes(ws),
                                          _stream(stream)))


def tdc_apply(x_in, delta, x_out, sums2=None, ws=None, n=None, stream=None):
    n = x_in.numel() if n is None else n
    _check("tdc_apply", lib().tdc_apply(_ptr(x_in), _ptr(delta), _ptr(x_out), n, _ptr(sums2),
                                        _ptr(ws), _nbytes(ws), _stream(stream)))


def tdc_apply_amax(x_in, delta, x_out, out_amax, sums2=None, ws=None, n=None, stream=None):
    """tdc_apply that also max-combines |x_out| into the device word out_amax."""
    n = x_in.numel() if n is None else n
    _check("tdc_apply_amax", lib().tdc_apply_amax(_ptr(x_in), _ptr(delta), _ptr(x_out), n,
                                                  _ptr(sums2), _ptr(out_amax), _ptr(ws),
                                                  _nbytes(ws), _stream(stream)))


def rel_err(y_q, y_ref, sums2, ws, n=None, stream=None):
    """sums2 <- {sum (y_q - y_ref)^2, sum y_ref^2} over bf16 device arrays."""
    n = y_q.numel() if n is None else n
    _check("rel_err", lib().rel_err(_ptr(y_q), _ptr(y_ref), n, _ptr(sums2), _ptr(ws),
                                    _nbytes(ws), _stream(stream)))


def delta_cosine(d_new, d_prev, sums3, ws, n=None, stream=None):
    """sums3 <- {sum d_new d_prev, sum d_new^2, sum d_prev^2} (bf16 device arrays)."""
    n = d_new.numel() if n is None else n
    _check("delta_cosine", lib().delta_cosine(_ptr(d_new), _ptr(d_prev), n, _ptr(sums3),
                                              _ptr(ws), _nbytes(ws), _stream(stream)))


# ------------------------------------------------------- host decisions --

def _host_array(a, dtype):
    """`a` as a C-contiguous numpy array of `dtype` (no copy when it already is)."""
    import numpy as np
    if isinstance(a, np.ndarray) and a.dtype == dtype and a.flags.c_contiguous:
        return a
    return np.ascontiguousarray(a, dtype=dtype)


def dmpq_mask(gamma_prev, alpha, beta, tau, L, J, out=None):
    """gamma_prev: float64 [L] or None; alpha/beta float32 [L*J]; returns the
    uint8 mask [L*J] (written into `out` when given)."""
    import numpy as np
    mask = np.zeros(L * J, dtype=np.uint8) if out is None else out
    if mask.dtype != np.uint8 or mask.size < L * J or not mask.flags.c_contiguous:
        raise ValueError("dmpq_mask: out must be a contiguous uint8 array of L*J entries")
    a = _host_array(alpha, np.float32)
    b = _host_array(beta, np.float32)
    if a.size < L * J or b.size < L * J:
        raise ValueError("dmpq_mask: alpha and beta need L*J entries")
    g = None if gamma_prev is None else _host_array(gamma_prev, np.float64)
    if g is not None and g.size < L:
        raise ValueError("dmpq_mask: gamma_prev needs L entries")
    _check("dmpq_mask", lib().dmpq_mask(None if g is None else g.ctypes.data, L, J,
                                        a.ctypes.data, b.ctypes.data, float(tau), mask.ctypes.data))
    return mask


def tdc_decide(t, d_prev, computed_prev, delta, out=None):
    import numpy as np
    d = _host_array(d_prev, np.float64)
    c = _host_array(computed_prev, np.uint8)
    if c.size < d.size:
        raise ValueError("tdc_decide: computed_prev needs one entry per block")
    skip = np.zeros(d.size, dtype=np.uint8) if out is None else out
    if skip.dtype != np.uint8 or skip.size < d.size or not skip.flags.c_contiguous:
        raise ValueError("tdc_decide: out must be a contiguous uint8 array, one entry per block")
    _check("tdc_decide", lib().tdc_decide(int(t), d.ctypes.data, c.ctypes.data, d.size, float(delta),
                                          skip.ctypes.data))
    return skip


def dmpq_fit(gamma, erel, J):
    """Per-linear (alpha, beta) float32 [L*J] from gamma [T, L] and erel
    [T, L*J] (host arrays; pairs gamma[t-1], erel[t])."""
    import numpy as np
    g = _host_array(gamma, np.float64)
    e = _host_array(erel, np.float64)
    if g.ndim != 2 or e.ndim != 2 or e.shape != (g.shape[0], g.shape[1] * J):
        raise ValueError("dmpq_fit: gamma must be [T, L] and erel [T, L*J]")
    T, L = g.shape
    alpha = np.zeros(L * J, np.float32)
    beta = np.zeros(L * J, np.float32)
    _check("dmpq_fit", lib().dmpq_fit(g.ctypes.data, e.ctypes.data, T, L, J, alpha.ctypes.data,
                                      beta.ctypes.data))
    return alpha, beta


def tdc_decide_cos(t, cos_prev, computed_prev, threshold, out=None):
    import numpy as np
    c = _host_array(cos_prev, np.float64)
    cp = _host_array(computed_prev, np.uint8)
    if cp.size < c.size:
        raise ValueError("tdc_decide_cos: computed_prev needs one entry per block")
    skip = np.zeros(c.size, dtype=np.uint8) if out is None else out
    if skip.dtype != np.uint8 or skip.size < c.size or not skip.flags.c_contiguous:
        raise ValueError("tdc_decide_cos: out must be a contiguous uint8 array, one entry per block")
    _check("tdc_decide_cos", lib().tdc_decide_cos(int(t), c.ctypes.data, cp.ctypes.data, c.size,
                                                  float(threshold), skip.ctypes.data))
    return skip


def cosine_from_sums(sums3):
    import numpy as np
    s = _host_array(sums3, np.float64)
    if s.size < 3:
        raise ValueError("cosine_from_sums: needs the three sums")
    return lib().qa_cosine_from_sums(s.ctypes.data)


def convert_check(op, first, out, count=None, stream=None):
    """Test-only: the library's element conversion `op` (0 E2M1, 1 E4M3
    scale, 2 bf16) of the float32 patterns first .. first + count - 1 into
    the device tensor out (u8, or int16 for bf16)."""
    count = out.numel() if count is None else count
    _check("qa_test_convert", lib().qa_test_convert(op, first, count, _ptr(out), _stream(stream)))


def stage_ab(design, iters, blocks, inp, out, stream=None):
    """Test/benchmark only: the compute stage of NVFP4 GEMM design 0, 1 or 2
    (qa_test_stage_ab) on the per-lane operands in `inp` (int32 [1024, 64])
    into `out` (float32 [1024, 256])."""
    _check("qa_test_stage_ab", lib().qa_test_stage_ab(design, iters, blocks, _ptr(inp), _ptr(out),
                                                      _stream(stream)))


def set_gemm_events(before, after):
    """Record raw hipEvent_t handles (ints) around every main GEMM kernel;
    (None, None) stops."""
    _check("qa_set_gemm_events", lib().qa_set_gemm_events(before, after))


def gamma_from_sums(sums2):
    import numpy as np
    s = _host_array(sums2, np.float64)
    if s.size < 2:
        raise ValueError("gamma_from_sums: needs the two sums")
    return lib().qa_gamma_from_sums(s.ctypes.data)


def rel_err_from_sums(sums2):
    import numpy as np
    s = _host_array(sums2, np.float64)
    if s.size < 2:
        raise ValueError("rel_err_from_sums: needs the two sums")
    return lib().qa_rel_err_from_sums(s.ctypes.data)


def rel_l2_from_sums(sums4):
    import numpy as np
    s = _host_array(sums4, np.float64)
    if s.size < 4:
        raise ValueError("rel_l2_from_sums: needs the four sums")
    return lib().qa_rel_l2_from_sums(s.ctypes.data)


# ------------------------------------------------- device-side step control --

# gate bits of qa_decide_step's flag bytes
ROUTE_NVFP4, ROUTE_INT8 = 1, 2
BLK_RUN0, BLK_RUN1, BLK_SKIP0, BLK_SKIP1 = 1, 2, 4, 8


def set_gate(flags, bits=0):
    """Gate every following call of this thread on the device byte `flags`
    (a uint8 tensor of one element, or a one-element slice): its kernels run
    only if (flags & bits) != 0.  set_gate(None) clears."""
    _check("qa_set_gate", lib().qa_set_gate(_ptr(flags), bits if flags is not None else 0))


class gate:
    """Context manager form of set_gate."""

    def __init__(self, flags, bits):
        self.flags, self.bits = flags, bits

    def __enter__(self):
        set_gate(self.flags, self.bits)

    def __exit__(self, *exc):
        set_gate(None)


def decide_step(sums, alpha, beta, tau, delta, L, J, t_ctr, bstate, d_prev, blk_flags, lin_flags,
                mask_out=None, skip_out=None, stream=None):
    """One timestep's DMPQ masks and TDC skips on the device (qa_decide_step)."""
    _check("qa_decide_step", lib().qa_decide_step(
        _ptr(sums), _ptr(alpha), _ptr(beta), tau, delta, L, J, _ptr(t_ctr), _ptr(bstate),
        _ptr(d_prev), _ptr(blk_flags), _ptr(lin_flags), _ptr(mask_out), _ptr(skip_out),
        _stream(stream)))
