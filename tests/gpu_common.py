"""Helpers shared by the GPU parity tests: exact decoding of 16-bit results,
ulp sizes and bitwise tensor comparison (no test functions here)."""
import numpy as np
import torch

import workloads as wl


def decode(t: torch.Tensor, dtype: str) -> np.ndarray:
    """bf16 or fp16 tensor (any device) -> exact fp64 values."""
    bits = wl.u16(t.cpu())
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp(v: np.ndarray, dtype: str) -> np.ndarray:
    """Unit in the last place of bf16 (8-bit significand) or fp16 (11-bit)
    at |v|, with the subnormal spacing below the smallest normal."""
    p, emin = (11, -14) if dtype == "fp16" else (8, -126)
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** emin)))
    return 2.0 ** (e - p + 1)


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Same dtype and bit-identical contents."""
    view = torch.int32 if a.dtype == torch.float32 else torch.int16
    return a.dtype == b.dtype and torch.equal(a.view(view), b.view(view))
