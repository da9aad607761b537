"""Helpers for the GPU parity tests (marshalling between NumPy and torch)."""
import numpy as np
import torch


def to_dev(a: np.ndarray, dev) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev)
    return torch.from_numpy(a).to(dev)


def to_host(t: torch.Tensor, dtype=None) -> np.ndarray:
    torch.cuda.synchronize()
    a = t.detach().cpu().numpy()
    if t.dtype == torch.int16:
        a = a.view(np.uint16)
    return a if dtype is None else a.astype(dtype)


def empty_f16(shape, dev):
    return torch.empty(shape, dtype=torch.int16, device=dev)


def ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in fp16 units in the last place between two fp16 bit arrays (finite values)."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + x)
    return np.abs(ordered(a_bits) - ordered(b_bits))
