"""Parity of the fused input prologue (gdn_forward_packed / gdn_forward_bidi_packed:
q, k, v read in place from a packed [B, T, 2 H d_k + H d_v] projection, q and k
L2-normalised and the gate logits activated inside the kernels) with the float64
oracle's prologue + recurrence, through the C ABI.  Every form is covered: the bf16
MFMA chunked kernel, the fp32 general chunked kernel, the scan and the bidirectional
form, with padded token strides and gaps between batch elements (the padding holds
NaN, so a read outside the packed rows would show)."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_recurrence_gdn_amd import inputs
from gated_deltanet_recurrence_gdn_amd import binding as gb
from gpu_util import TOL, host, parity_by_head

pytestmark = pytest.mark.gpu


def make(B, T, H, dk, dv, io, seed=0, pad=0, gap=0, a_mean=0.0, state=False):
    x = inputs.make_packed_inputs(B, T, H, dk, dv, io, seed=seed, pad=pad, gap=gap, a_mean=a_mean)
    s0 = None
    if state:
        g = torch.Generator().manual_seed(seed + 3000)
        s0 = 0.3 * torch.randn((B, H, dv, dk), generator=g, dtype=torch.float32)
    return x, s0


def to_dev(x):
    """The packed view on the device with the buffer's strides kept."""
    buf = x["qkv_buf"].cuda()
    T, W = x["qkv"].shape[1], x["qkv"].shape[2]
    return buf[:, :T, :W], x["beta_logit"].cuda(), x["decay_logit"].cuda()


def run(x, s0, B, H, dk, dv, io, chunk, max_T=None):
    qkv, bl, dl = to_dev(x)
    T = qkv.shape[1]
    g = gb.GDN(B, H, dk, dv, io, max_T=max_T or T)
    out, st = g.forward_packed(qkv, bl, dl, state_in=None if s0 is None else s0.cuda(), chunk_len=chunk)
    torch.cuda.synchronize()
    g.close()
    return out, st


def check(out, st, x, s0, H, dk, dv, io, what):
    o64, s64 = oracle.forward_packed(x["qkv"], x["beta_logit"], x["decay_logit"], H, dk, dv, state_in=s0)
    r1, r2 = oracle.rel_l2(host(out), o64), oracle.rel_l2(host(st), s64)
    print(f"{what}: rel-L2 out {r1:.3e} state {r2:.3e}")
    assert r1 <= TOL[io] and r2 <= TOL[io], (r1, r2)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (32, 128), (128, 32)])
def test_mfma_chunked_padded_strides(dk, dv):
    B, T, H = 2, 301, 3
    x, s0 = make(B, T, H, dk, dv, "bf16", seed=dk + dv, pad=24, gap=5, state=True)
    out, st = run(x, s0, B, H, dk, dv, "bf16", 64)
    check(out, st, x, s0, H, dk, dv, "bf16", f"mfma dk={dk} dv={dv}")


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_mfma_lengths(T):
    B, H, d = 1, 8, 64
    x, s0 = make(B, T, H, d, d, "bf16", seed=T, pad=8, state=True)
    out, st = run(x, s0, B, H, d, d, "bf16", 64)
    check(out, st, x, s0, H, d, d, "bf16", f"mfma T={T}")


@pytest.mark.parametrize("io,chunk,dk,dv", [("fp32", 32, 64, 32), ("fp32", 128, 16, 64), ("bf16", 16, 16, 16),
                                            ("fp32", 64, 128, 128)])
def test_general_chunked(io, chunk, dk, dv):
    B, T, H = 2, 157, 2
    x, s0 = make(B, T, H, dk, dv, io, seed=chunk + dk, pad=8, gap=3, state=True)
    out, st = run(x, s0, B, H, dk, dv, io, chunk)
    check(out, st, x, s0, H, dk, dv, io, f"general {io} C={chunk} dk={dk} dv={dv}")


@pytest.mark.parametrize("io,dk,dv", [("fp32", 64, 32), ("bf16", 128, 128), ("fp32", 16, 16), ("bf16", 32, 64)])
def test_scan(io, dk, dv):
    B, T, H = 2, 133, 3
    x, s0 = make(B, T, H, dk, dv, io, seed=dk * 3 + dv, pad=8, gap=2, state=True)
    out, st = run(x, s0, B, H, dk, dv, io, 1)
    check(out, st, x, s0, H, dk, dv, io, f"scan {io} dk={dk} dv={dv}")


@pytest.mark.parametrize("io,chunk", [("bf16", 64), ("fp32", 1), ("fp32", 32)])
def test_bidi_and_reversal(io, chunk):
    B, T, H, d = 1, 190, 2, 64
    x, _ = make(B, T, H, d, d, io, seed=5 + chunk, pad=8)
    qkv, bl, dl = to_dev(x)
    g = gb.GDN(B, H, d, d, io, max_T=T, bidi=True)
    out = g.forward_bidi_packed(qkv, bl, dl, chunk_len=chunk)
    # the reversed inputs (a reversed view of the same buffer keeps the packed strides)
    out_r = g.forward_bidi_packed(torch.flip(qkv, dims=[1]).contiguous(), torch.flip(bl, dims=[1]).contiguous(),
                                  torch.flip(dl, dims=[1]).contiguous(), chunk_len=chunk)
    torch.cuda.synchronize()
    g.close()
    assert torch.equal(torch.flip(out_r, dims=[1]), out)
    ob = oracle.bidi_packed(x["qkv"], x["beta_logit"], x["decay_logit"], H, d, d)
    r = oracle.rel_l2(host(out), ob)
    print(f"bidi {io} C={chunk}: rel-L2 {r:.3e}")
    assert r <= TOL[io]


@pytest.mark.parametrize("chunk", [1, 64])
def test_streaming_split_bit_identical(chunk):
    """Calls over consecutive token ranges (chunk-aligned for the chunked form) with the
    state carried reproduce one call bit for bit; the prologue is per token, so the
    split does not touch it."""
    B, T, H, d = 1, 320, 4, 128
    x, s0 = make(B, T, H, d, d, "bf16", seed=77, pad=16, state=True)
    qkv, bl, dl = to_dev(x)
    g = gb.GDN(B, H, d, d, "bf16", max_T=T)
    o1, st1 = g.forward_packed(qkv, bl, dl, state_in=s0.cuda(), chunk_len=chunk)
    state = s0.cuda().clone()
    outs = []
    for a_, b_ in [(0, 128), (128, 192), (192, 320)]:
        o, _ = g.forward_packed(qkv[:, a_:b_], bl[:, a_:b_].contiguous(), dl[:, a_:b_].contiguous(),
                                state_in=state, state_out=state, chunk_len=chunk)
        outs.append(o)
    torch.cuda.synchronize()
    g.close()
    assert torch.equal(torch.cat(outs, dim=1), o1) and torch.equal(state, st1)


@pytest.mark.parametrize("chunk", [1, 64, 32])
def test_zero_query_rows_give_zero_outputs(chunk):
    """A zero q row stays zero after normalisation (max(||q||, 1e-12)), so its output
    is exactly zero; zero k rows write nothing.  No inf or NaN comes out of the
    inverse norms."""
    io = "fp32" if chunk == 32 else "bf16"
    B, T, H, d = 1, 150, 2, 64
    x, s0 = make(B, T, H, d, d, io, seed=9, state=True)
    zq = [0, 5, 64, 149]
    zk = [3, 70, 100]
    for t in zq:
        x["qkv_buf"][:, t, :H * d] = 0
    for t in zk:
        x["qkv_buf"][:, t, H * d:2 * H * d] = 0
    out, st = run(x, s0, B, H, d, d, io, chunk)
    assert bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(st).all())
    assert bool((out[:, zq] == 0).all())
    check(out, st, x, s0, H, d, d, io, f"zero rows C={chunk}")


@pytest.mark.parametrize("chunk", [1, 64])
def test_extreme_logits(chunk):
    """Logits of +-40 (b, a saturate at 0 or 1 in fp32) and 0: no overflow, oracle parity."""
    B, T, H, d = 1, 130, 2, 64
    x, s0 = make(B, T, H, d, d, "bf16", seed=21, state=True)
    g = torch.Generator().manual_seed(4)
    pick = torch.randint(0, 3, (B, T, H), generator=g)
    vals = torch.tensor([-40.0, 0.0, 40.0])
    x["beta_logit"] = vals[pick].contiguous()
    x["decay_logit"] = vals[torch.randint(0, 3, (B, T, H), generator=g)].contiguous()
    out, st = run(x, s0, B, H, d, d, "bf16", chunk)
    assert bool(torch.isfinite(out.float()).all())
    check(out, st, x, s0, H, d, d, "bf16", f"extreme logits C={chunk}")


def test_full_size_all_heads():
    """The bench shape (B=2, H=32, T=32760, d=128, decay logits N(2,1)) from a packed
    [B, T, 12288] bf16 projection on the MFMA path: every head vs the oracle, per head
    and per edge chunk."""
    w = inputs.WORKLOADS["batched_bf16_d128"]
    x, _ = make(w.B, w.T, w.H, w.dk, w.dv, "bf16", seed=0, a_mean=w.a_mean)
    qkv, bl, dl = to_dev(x)
    g = gb.GDN(w.B, w.H, w.dk, w.dv, "bf16", max_T=w.T)
    out, st = g.forward_packed(qkv, bl, dl, chunk_len=64)
    torch.cuda.synchronize()
    g.close()
    del qkv, bl, dl
    assert bool(torch.isfinite(out.float()).all())
    o64, s64 = oracle.forward_packed(x["qkv"], x["beta_logit"], x["decay_logit"], w.H, w.dk, w.dv)
    parity_by_head("packed full size", out, o64, TOL["bf16"], st, s64)


@pytest.mark.parametrize("io,chunk", [("bf16", 64), ("bf16", 1), ("fp32", 32)])
def test_normalisation_makes_scale_irrelevant(io, chunk):
    """q and k are L2-normalised inside the kernels, so scaling every q row by 2^-9 and
    every k row by 2^7 (exact in bf16 and fp32) leaves out and the state unchanged up to
    rounding: the norms, and the exponents of the decay factors that carry 1/||k||, can
    round differently, which may move a few bf16 outputs by one unit (a missing
    normalisation would show as a factor of 2^9)."""
    B, T, H, d = 1, 200, 2, 128 if io == "bf16" else 64
    x, s0 = make(B, T, H, d, d, io, seed=31, pad=8, state=True)
    out, st = run(x, s0, B, H, d, d, io, chunk)
    y = dict(x)
    buf = x["qkv_buf"].clone()
    buf[:, :, :H * d] *= 2.0 ** -9
    buf[:, :, H * d:2 * H * d] *= 2.0 ** 7
    y["qkv_buf"] = buf
    out2, st2 = run(y, s0, B, H, d, d, io, chunk)
    r1 = oracle.rel_l2(host(out2), host(out))
    r2 = oracle.rel_l2(host(st2), host(st))
    print(f"{io} C={chunk}: rel-L2 scaled vs unscaled out {r1:.3e} state {r2:.3e}")
    tol = 1e-3 if io == "bf16" else 1e-6
    assert r1 <= tol and r2 <= tol
