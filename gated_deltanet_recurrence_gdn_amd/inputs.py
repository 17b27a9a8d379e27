"""Seeded synthetic inputs for the GDN recurrence.

This module holds no arithmetic of the recurrence itself: it only draws random
numbers and prepares them the way the model would hand them to the recurrence
(unit-norm q/k per token, sigmoid write strength b, exp(-softplus) decay a), so
that the oracle and the device library both consume the same values.

Workloads.  The pages' workload is 480x832 video in a SANA video DiT (diffusers
LongSANA PR page, "Code snap": height=480, width=832); the shapes below use
30x52 = 1560 latent tokens per frame, flattened frame-major in raster order
(T = frames * 1560).  Standard normal draws stand in for real activations; no
dataset is used or needed.

Recipe: one torch CPU ``Generator`` seeded with ``seed``, float32 draws in the
order q, k, v, x_b, x_a with shapes [B,T,H,d_k], [B,T,H,d_k], [B,T,H,d_v],
[B,T,H], [B,T,H]; q and k are divided by max(||x||_2, 1e-12) over the last
axis; b = sigmoid(x_b + b_mean), a = exp(-softplus(x_a + a_mean)); q, k, v are
then rounded to bf16 or to FP8 E4M3 (round-to-nearest-even) for those I/O types.
beta and decay stay float32.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import torch

TOKENS_PER_FRAME = 30 * 52  # 480x832 video at a 16x spatial reduction

# q, k, v element types: fp8 is OCP FP8 E4M3 (torch.float8_e4m3fn, round to nearest
# even from fp32; every draw here is far inside its +-448 range).
IO_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    io: str  # "fp32" | "bf16"
    chunk_len: int = 64
    calls: int = 1  # streaming: T is split into `calls` equal calls
    bidi: bool = False
    a_mean: float = 0.0
    b_mean: float = 0.0
    note: str = ""

    @property
    def token_heads(self) -> int:
        return self.B * self.H * self.T


WORKLOADS = {
    "causal_fp32_tiny": Workload(
        "causal_fp32_tiny", B=1, H=2, T=64, dk=16, dv=16, io="fp32", chunk_len=1,
        note="causal, fp32, zero initial state"),
    "causal_bf16_d64": Workload(
        "causal_bf16_d64", B=1, H=16, T=3 * TOKENS_PER_FRAME, dk=64, dv=64, io="bf16",
        note="3 latent frames x 30x52 tokens, one call"),
    "streaming_bf16_d128": Workload(
        "streaming_bf16_d128", B=1, H=20, T=5 * 3 * TOKENS_PER_FRAME, dk=128, dv=128, io="bf16",
        calls=5, note="5 calls of 4680 tokens, fp32 state carried between calls"),
    "bidi_bf16_d128": Workload(
        "bidi_bf16_d128", B=1, H=20, T=21 * TOKENS_PER_FRAME, dk=128, dv=128, io="bf16",
        bidi=True, note="21 latent frames, causal + reversed causal scan"),
    "batched_bf16_d128": Workload(
        "batched_bf16_d128", B=2, H=32, T=21 * TOKENS_PER_FRAME, dk=128, dv=128, io="bf16",
        a_mean=2.0, note="guidance pair, decay a = exp(-softplus(N(2,1)))"),
}


def make_inputs(B: int, T: int, H: int, dk: int, dv: int, io: str = "bf16", seed: int = 0,
                a_mean: float = 0.0, b_mean: float = 0.0) -> dict:
    """Draw one seeded input set on the CPU.  Returns torch CPU tensors
    q, k [B,T,H,dk] and v [B,T,H,dv] in the I/O dtype, beta and decay [B,T,H] float32."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = torch.randn((B, T, H, dk), generator=g, dtype=torch.float32)
    k = torch.randn((B, T, H, dk), generator=g, dtype=torch.float32)
    v = torch.randn((B, T, H, dv), generator=g, dtype=torch.float32)
    xb = torch.randn((B, T, H), generator=g, dtype=torch.float32)
    xa = torch.randn((B, T, H), generator=g, dtype=torch.float32)
    q = torch.nn.functional.normalize(q, p=2.0, dim=-1, eps=1e-12)
    k = torch.nn.functional.normalize(k, p=2.0, dim=-1, eps=1e-12)
    beta = torch.sigmoid(xb + b_mean)
    decay = torch.exp(-torch.nn.functional.softplus(xa + a_mean))
    dt = IO_DTYPES[io]
    return {"q": q.to(dt).contiguous(), "k": k.to(dt).contiguous(), "v": v.to(dt).contiguous(),
            "beta": beta.contiguous(), "decay": decay.contiguous()}


def make_packed_inputs(B: int, T: int, H: int, dk: int, dv: int, io: str = "bf16", seed: int = 0,
                       a_mean: float = 0.0, b_mean: float = 0.0, pad: int = 0, gap: int = 0) -> dict:
    """Raw inputs of the fused prologue, drawn on the CPU: the projection output
    before any normalisation and the gate logits.

    ``qkv_buf`` is a [B, T + gap, W + pad] tensor in the I/O dtype with W = 2 H d_k + H d_v;
    ``qkv`` is its [B, T, W] view (token stride W + pad, batch stride (T + gap)(W + pad)
    elements), holding q (H d_k columns), k (H d_k) and v (H d_v), standard normal.  The
    pad columns and gap tokens hold NaN: they are never part of the input.
    ``beta_logit`` = x_b + b_mean and ``decay_logit`` = x_a + a_mean, float32 [B, T, H],
    with x_b, x_a standard normal.  Draw order: q, k, v, x_b, x_a as in make_inputs."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = torch.randn((B, T, H * dk), generator=g, dtype=torch.float32)
    k = torch.randn((B, T, H * dk), generator=g, dtype=torch.float32)
    v = torch.randn((B, T, H * dv), generator=g, dtype=torch.float32)
    xb = torch.randn((B, T, H), generator=g, dtype=torch.float32)
    xa = torch.randn((B, T, H), generator=g, dtype=torch.float32)
    dt = IO_DTYPES[io]
    W = 2 * H * dk + H * dv
    buf = torch.full((B, T + gap, W + pad), float("nan"), dtype=dt)
    buf[:, :T, :W] = torch.cat([q, k, v], dim=-1).to(dt)
    return {"qkv_buf": buf, "qkv": buf[:, :T, :W], "beta_logit": (xb + b_mean).contiguous(),
            "decay_logit": (xa + a_mean).contiguous()}


def make_workload(w: Workload | str, seed: int = 0, T: int | None = None) -> dict:
    """Inputs for a named workload; ``T`` overrides the sequence length (a prefix-sized
    sample of the same distribution, drawn from the same seed)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    return make_inputs(w.B, w.T if T is None else T, w.H, w.dk, w.dv, w.io, seed, w.a_mean, w.b_mean)


def sha256(inputs: dict) -> str:
    """SHA256 over the raw bytes of q, k, v, beta, decay (in that order)."""
    h = hashlib.sha256()
    for name in ("q", "k", "v", "beta", "decay"):
        t = inputs[name].contiguous()
        h.update(t.view(torch.uint8).numpy().tobytes() if t.dtype != torch.bfloat16
                 else t.view(torch.int16).numpy().tobytes())
    return h.hexdigest()
