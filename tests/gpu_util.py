"""GPU-test utilities: moving bf16 bit arrays between numpy and torch."""
from __future__ import annotations

import sys

import numpy as np
import torch


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def f64_to_bits(x: np.ndarray) -> np.ndarray:
    """Exactly-representable bf16 values (float64) -> bit patterns."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def i32(x) -> torch.Tensor:
    return torch.tensor(list(x), dtype=torch.int32, device="cuda")
