"""Device upload / download helpers for the GPU parity tests."""
from __future__ import annotations

import numpy as np
import torch

TORCH = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16,
         "int32": torch.int32, "int8": torch.int8}


def to_dev(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def strided_buffers(xs, dtype, offsets, device="cuda"):
    """Rank buffers carved from one allocation at the given element offsets
    (to give the buffers chosen 16-byte phases).  Returns (views, backing)."""
    L = xs[0].size
    pad = 64
    P = len(xs)
    stride = (L + pad + 15) // 16 * 16  # keeps every rank's base on one 16-byte phase
    backing = torch.zeros(P * stride + pad, dtype=TORCH[dtype], device=device)
    views = []
    for r, x in enumerate(xs):
        off = r * stride + offsets[r]
        v = backing.narrow(0, off, L)
        v.copy_(to_dev(x, dtype, device))
        views.append(v)
    return views, backing
