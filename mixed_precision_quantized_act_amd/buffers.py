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
