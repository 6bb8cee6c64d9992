"""Helpers shared by the GPU tests: moving bf16/uint32 bit patterns between
NumPy and torch GPU tensors, and the comparison metrics.  No method arithmetic."""
from __future__ import annotations

import numpy as np
import torch


def gpu_available() -> bool:
    return torch.cuda.is_available()


def to_bf16(u16: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).to(device)


def to_i32(u32: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u32).view(np.int32)).to(device)


def to_f32(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits32(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy().view(np.uint32)


def bf16_values(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rel_fro(y: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(y - ref) / den) if den > 0 else float(np.linalg.norm(y))


def say(*args):
    print("[case]", *args, flush=True)
