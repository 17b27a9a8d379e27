"""Helpers for the GPU parity tests: move seeded inputs to the device, call the
library through the C ABI (binding.GDN), compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle

# rel-L2 bars against the float64 oracle, by I/O dtype.  The oracle reads the very
# bf16 / FP8 values the GPU receives, so the bar covers only the kernel arithmetic
# and the output rounding, which are the same for bf16 and FP8 inputs.
TOL = {"fp32": 1e-5, "bf16": 1e-2, "fp8": 1e-2}


def dev(x: dict, device="cuda:0") -> dict:
    return {k: v.to(device) for k, v in x.items()}


def host(t) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy().astype(np.float64)


def slice_tokens(x: dict, a: int, b: int) -> dict:
    return {k: v[:, a:b].contiguous() for k, v in x.items()}


def reverse_tokens(x: dict) -> dict:
    return {k: torch.flip(v, dims=[1]).contiguous() for k, v in x.items()}


def rel(a, b) -> float:
    return oracle.rel_l2(host(a) if isinstance(a, torch.Tensor) else a, b)
