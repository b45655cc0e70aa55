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
    "qlinear_int8": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _I64,
                                    ctypes.c_int, ctypes.c_int, _P, _SZ, _P]),
    "qlinear_layer_workspace": (_SZ, [ctypes.c_int, _I64, _I64, _I64]),
    "qlinear": (ctypes.c_int, [ctypes.c_int, _P, _I64, _P, ctypes.c_uint32, _P, _P, _P, _I64, _I64,
                               _I64, _P, _P, _I64, ctypes.c_int, ctypes.c_int, _P, _SZ, _P]),
    "reduce_workspace": (_SZ, [_I64]),
    "block_gamma": (ctypes.c_int, [_P, _P, _I64, _P, _P, _SZ, _P]),
    "tdc_update": (ctypes.c_int, [_P, _P, _P, _P, _I64, _P, _P, _SZ, _P]),
    "tdc_apply": (ctypes.c_int, [_P, _P, _P, _I64, _P, _P, _SZ, _P]),
    "dmpq_mask": (ctypes.c_int, [_P, ctypes.c_int, ctypes.c_int, _P, _P, ctypes.c_double, _P]),
    "tdc_decide": (ctypes.c_int, [ctypes.c_int, _P, _P, ctypes.c_int, ctypes.c_double, _P]),
    "qa_set_gemm_events": (ctypes.c_int, [_P, _P]),
    "qa_gamma_from_sums": (ctypes.c_double, [_P]),
    "qa_rel_l2_from_sums": (ctypes.c_double, [_P]),
}

EXPORTS = tuple(_SIGS)


def lib():
    """The loaded library (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libqact.so is not built at {LIB_PATH}; run "
                              "python -m mixed_precision_quantized_act_amd.build")
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
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


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
                 ws=None, ldy=None, stream=None):
    ldy = y.stride(0) if ldy is None else ldy
    _check("qlinear_int8", lib().qlinear_int8(
        _ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s), _ptr(w_ts), M, N, K, _ptr(bias), _ptr(y),
        ldy, out, epi, _ptr(ws), _nbytes(ws), _stream(stream)))


def qlinear_layer_workspace(fmt, M, N, K):
    return lib().qlinear_layer_workspace(fmt, M, N, K)


def qlinear(fmt, x, x_ts, w_q, w_s, w_ts, y, M, N, K, bias=None, out=OUT_BF16, epi=EPI_NONE,
            flags=0, ws=None, ldx=None, ldy=None, stream=None):
    ldx = x.stride(0) if ldx is None else ldx
    ldy = y.stride(0) if ldy is None else ldy
    _check("qlinear", lib().qlinear(
        fmt, _ptr(x), ldx, _ptr(x_ts), flags, _ptr(w_q), _ptr(w_s), _ptr(w_ts), M, N, K,
        _ptr(bias), _ptr(y), ldy, out, epi, _ptr(ws), _nbytes(ws), _stream(stream)))


# ------------------------------------------------------------- Gamma / TDC --

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


# ------------------------------------------------------- host decisions --

def dmpq_mask(gamma_prev, alpha, beta, tau, L, J):
    """gamma_prev: float64 numpy [L] or None; alpha/beta float32 [L*J]."""
    import numpy as np
    mask = np.zeros(L * J, dtype=np.uint8)
    a = np.ascontiguousarray(alpha, dtype=np.float32)
    b = np.ascontiguousarray(beta, dtype=np.float32)
    g = None if gamma_prev is None else np.ascontiguousarray(gamma_prev, dtype=np.float64)
    _check("dmpq_mask", lib().dmpq_mask(None if g is None else g.ctypes.data_as(_P), L, J,
                                        a.ctypes.data_as(_P), b.ctypes.data_as(_P), float(tau),
                                        mask.ctypes.data_as(_P)))
    return mask


def tdc_decide(t, d_prev, computed_prev, delta):
    import numpy as np
    d = np.ascontiguousarray(d_prev, dtype=np.float64)
    c = np.ascontiguousarray(computed_prev, dtype=np.uint8)
    skip = np.zeros(len(d), dtype=np.uint8)
    _check("tdc_decide", lib().tdc_decide(int(t), d.ctypes.data_as(_P), c.ctypes.data_as(_P),
                                          len(d), float(delta), skip.ctypes.data_as(_P)))
    return skip


def set_gemm_events(before, after):
    """Record raw hipEvent_t handles (ints) around every main GEMM kernel;
    (None, None) stops."""
    _check("qa_set_gemm_events", lib().qa_set_gemm_events(before, after))


def gamma_from_sums(sums2):
    import numpy as np
    s = np.ascontiguousarray(sums2, dtype=np.float64)
    return lib().qa_gamma_from_sums(s.ctypes.data_as(_P))


def rel_l2_from_sums(sums4):
    import numpy as np
    s = np.ascontiguousarray(sums4, dtype=np.float64)
    return lib().qa_rel_l2_from_sums(s.ctypes.data_as(_P))
