"""Upload seeded host inputs (bf16 bits, int32 tables) to a HIP device via torch.

Data movement only; shared by the GPU tests and the benchmark.
"""
from __future__ import annotations

import numpy as np
import torch


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on `device` (bit-exact)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def fp8_tensor(codes: np.ndarray, device) -> torch.Tensor:
    """uint8 E4M3 codes -> torch.float8_e4m3fn tensor on `device` (bit-exact)."""
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).to(device).view(torch.float8_e4m3fn)


def int32_tensor(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def f32_tensor(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
