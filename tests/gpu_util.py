"""Host <-> device helpers for the GPU parity tests (bits travel unchanged)."""

import numpy as np
import torch

import oracle


def to_dev(a: np.ndarray, bf16: bool = False) -> torch.Tensor:
    """numpy -> device tensor with the same bytes (uint16 -> int16, or bfloat16 if bf16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).cuda()
        return t.view(torch.bfloat16) if bf16 else t
    return torch.from_numpy(a).cuda()


def bits(t: torch.Tensor) -> np.ndarray:
    """2-byte device tensor -> uint16 numpy bits."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def vals(a: np.ndarray) -> np.ndarray:
    """uint16 bf16 bits or float32 -> float64 values."""
    return a.astype(np.float64) if a.dtype == np.float32 else oracle.bf16_bits_to_f64(a)


def rel_fro(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    """Relative Frobenius error per slot (0 where both are zero)."""
    d = np.sqrt(np.sum((got - want) ** 2, axis=(1, 2)))
    n = np.sqrt(np.sum(want ** 2, axis=(1, 2)))
    return np.where(n > 0, d / np.where(n > 0, n, 1), d)
