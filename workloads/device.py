"""Copies of the seeded host inputs to a HIP device (torch tensors).

bf16 bit patterns (np.uint16) become torch.bfloat16 tensors with the same bits;
everything else keeps its dtype.  Nothing here computes any part of the selector.
"""
from __future__ import annotations

import numpy as np
import torch


def to_dev(x: np.ndarray, device="cuda") -> torch.Tensor:
    if x.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def upload(inp, device="cuda") -> dict:
    return {
        "logits": to_dev(inp.logits, device),
        "hidden": to_dev(inp.hidden, device),
        "prev_token": torch.from_numpy(inp.prev_token.astype(np.int32)).to(device),
        "A": to_dev(inp.A, device),
        "B": to_dev(inp.B, device),
        "W_h": to_dev(inp.W_h, device),
    }
