"""Helpers of the GPU tests: numpy <-> device tensors with the same bytes,
and the relative Frobenius error used for GEMM outputs."""
import numpy as np

_VIEW = {np.uint16: np.int16}


def torch():
    import torch as t
    return t


def dev(a):
    """numpy array -> CUDA tensor holding the same bytes."""
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return t.from_numpy(a.copy()).cuda()


def host(t, dtype=None):
    """CUDA tensor -> numpy (uint16 for 16-bit integer/bf16 data)."""
    tt = torch()
    if t.dtype == tt.bfloat16:
        t = t.view(tt.int16)
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a if dtype is None else a.view(dtype)


def rel_fro(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return np.linalg.norm(y - ref) / (den if den else 1.0)


def sample_rows(M, n, seed, tile=256):
    """Sorted distinct rows: random ones, the first, and the ragged last tile."""
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(M, min(n, M), replace=False).tolist())
    pick |= {0, M - 1}
    last = (M - 1) // tile * tile
    pick |= set(range(last, min(last + 8, M)))
    return np.array(sorted(pick))
