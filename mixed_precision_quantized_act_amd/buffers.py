"""Device buffers in the library's layouts (allocation only, via torch)."""


def _torch():
    import torch
    return torch


def workspace(nbytes, device="cuda"):
    """Caller-owned device scratch of at least ``nbytes`` bytes (16-aligned)."""
    torch = _torch()
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def empty_nvfp4(rows, K, device="cuda"):
    """(codes u8 [rows, K/2], scales u8 [rows, K/16], tscale f32 [1])."""
    torch = _torch()
    return (torch.empty((rows, K // 2), dtype=torch.uint8, device=device),
            torch.empty((rows, K // 16), dtype=torch.uint8, device=device),
            torch.empty((1,), dtype=torch.float32, device=device))


def empty_int8_act(rows, K, device="cuda"):
    """(q i8 [rows, K], scale f32 [rows])."""
    torch = _torch()
    return (torch.empty((rows, K), dtype=torch.int8, device=device),
            torch.empty((rows,), dtype=torch.float32, device=device))


def empty_int8_planes(N, K, device="cuda"):
    """Device buffer for an NVFP4 weight's int8 digit planes
    (int8_weight_planes), 256-byte aligned."""
    from ._lib import int8_weight_planes_bytes
    torch = _torch()
    nbytes = int8_weight_planes_bytes(N, K)
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + nbytes]
