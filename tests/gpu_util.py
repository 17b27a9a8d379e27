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


def edge_slices(T: int, chunk: int = 64):
    """Token ranges where a localized error would hide in a whole-tensor norm: the
    first chunk (the reverse sweep's final partial chunk in the bidirectional form)
    and the final partial chunk (the last chunk if T is a multiple of `chunk`)."""
    r = T % chunk or chunk
    return [("first chunk", slice(0, min(chunk, T))), ("final partial chunk", slice(T - r, T))]


def parity_by_head(label: str, out, o64: np.ndarray, tol: float, st=None, s64=None, chunk: int = 64):
    """Compare every (b, h) separately, and each head's first and final partial chunk,
    besides the whole tensor: a wrong head, tile or tail cannot be diluted by the rest.
    out [B, T, H, d_v] (device or host), o64 the oracle's; st / s64 [B, H, d_v, d_k]."""
    x = host(out) if isinstance(out, torch.Tensor) else out
    B, T, H, _ = x.shape
    worst = {"whole": oracle.rel_l2(x, o64)}
    where = {"whole": None}
    for b in range(B):
        for h in range(H):
            cand = [("head", slice(0, T))] + edge_slices(T, chunk)
            for name, sl in cand:
                r = oracle.rel_l2(x[b, sl, h], o64[b, sl, h])
                if r > worst.get(name, -1.0):
                    worst[name], where[name] = r, (b, h)
    if st is not None:
        xs = host(st) if isinstance(st, torch.Tensor) else st
        worst["state"] = oracle.rel_l2(xs, s64)
        for b in range(B):
            for h in range(H):
                r = oracle.rel_l2(xs[b, h], s64[b, h])
                if r > worst.get("state per head", -1.0):
                    worst["state per head"], where["state per head"] = r, (b, h)
    msg = ", ".join(f"{k} {v:.3e}" + (f" at (b, h) = {where[k]}" if where.get(k) else "") for k, v in worst.items())
    print(f"{label}: worst rel-L2 {msg}", flush=True)
    bad = {k: v for k, v in worst.items() if not v <= tol}
    assert not bad, f"{label}: rel-L2 above {tol:.0e}: {bad}"
    return worst
