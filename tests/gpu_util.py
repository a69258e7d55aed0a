"""Helpers shared by the GPU parity tests (no arithmetic of the method)."""
import numpy as np
import torch

CANARY = 0x5A


def bits_to_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def tensor_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor (any device, any strides)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def padded(rows: int, cols: int, ld: int, dtype, device="cuda", fill=CANARY):
    """(storage [rows, ld], view [rows, cols]) with the padding filled by a canary byte."""
    store = torch.empty((rows, ld), dtype=dtype, device=device)
    store.view(torch.uint8).fill_(fill)
    return store, store[:, :cols]


def padded_copy(src: torch.Tensor, ld: int) -> torch.Tensor:
    """Copy of 2-D src into storage with leading dimension ld (padding = canary)."""
    store, view = padded(src.shape[0], src.shape[1], ld, src.dtype, src.device)
    view.copy_(src)
    return view


def canary_intact(store: torch.Tensor, cols: int) -> bool:
    pad = store[:, cols:].contiguous().view(torch.uint8)
    return bool((pad == CANARY).all().item()) if pad.numel() else True


def round_up(n: int, m: int) -> int:
    return (n + m - 1) // m * m


def random_codes(rng, shape) -> np.ndarray:
    return rng.integers(-127, 128, size=shape).astype(np.int8)


def special_rows_bf16(rng, rows, cols, std=1.0):
    """Gaussian bf16 bits with a few structured rows: all zero, subnormal-only,
    a single outlier, and exact-tie values with a power-of-two scale."""
    x = (rng.standard_normal((rows, cols)) * std).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 pattern is fine here
    if rows > 0:
        bits[0] = 0
    if rows > 1:
        bits[1] = rng.integers(0, 0x80, size=cols).astype(np.uint16) | (
            rng.integers(0, 2, size=cols).astype(np.uint16) << 15)
    if rows > 2 and cols > 1:
        bits[2] = 0x3F80  # 1.0
        bits[2, cols // 2] = 0x4400  # 512.0
    if rows > 3:
        vals = (np.arange(cols) % 254 - 127 + 0.5).astype(np.float32)
        vals[0] = 127.0
        bits[3] = (vals.view(np.uint32) >> 16).astype(np.uint16)
    return bits
