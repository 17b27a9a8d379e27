"""Parity of the general chunked kernel (fp32 arithmetic; chunk lengths 16, 32, 64,
128; head dims 16-128; fp32 or bf16 I/O) with the float64 oracle, through the C ABI.

The bf16 chunk_len = 64 requests with d_k, d_v >= 32 go to the MFMA kernel and are
covered by test_gpu_chunk.py; everything here runs on the general kernel."""
import pytest
import torch

import oracle
from gated_deltanet_recurrence_gdn_amd import inputs
from gated_deltanet_recurrence_gdn_amd import binding as gb
from gpu_util import TOL, dev, rel, reverse_tokens, slice_tokens

pytestmark = pytest.mark.gpu


def make(B, T, H, dk, dv, io, seed=0, a_mean=0.0, state=False):
    x = inputs.make_inputs(B, T, H, dk, dv, io, seed=seed, a_mean=a_mean)
    s0 = None
    if state:
        g = torch.Generator().manual_seed(seed + 2000)
        s0 = 0.3 * torch.randn((B, H, dv, dk), generator=g, dtype=torch.float32)
    return x, s0


def run(x, io, chunk, s0=None):
    B, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    g = gb.GDN(B, H, dk, dv, io, max_T=T)
    d = dev(x)
    out, st = g.forward(d["q"], d["k"], d["v"], d["beta"], d["decay"],
                        state_in=None if s0 is None else s0.cuda(), chunk_len=chunk)
    torch.cuda.synchronize()
    g.close()
    return out, st


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_tiny_fp32_workload_chunked(chunk):
    """B=1, H=2, T=64, d=16, fp32 I/O, zero initial state."""
    x = inputs.make_workload("causal_fp32_tiny")
    out, st = run(x, "fp32", chunk)
    o64, s64 = oracle.forward(**x)
    r1, r2 = rel(out, o64), rel(st, s64)
    print(f"chunk {chunk}: rel-L2 out {r1:.3e} state {r2:.3e}")
    assert r1 <= TOL["fp32"] and r2 <= TOL["fp32"]


@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (128, 128), (64, 16), (16, 128)])
def test_fp32_dims_ragged_with_state(chunk, dk, dv):
    x, s0 = make(2, 301, 3, dk, dv, "fp32", seed=chunk + dk + 3 * dv, state=True)
    out, st = run(x, "fp32", chunk, s0)
    o64, s64 = oracle.forward(**x, state_in=s0)
    r1, r2 = rel(out, o64), rel(st, s64)
    print(f"C={chunk} dk={dk} dv={dv}: rel-L2 out {r1:.3e} state {r2:.3e}")
    assert r1 <= TOL["fp32"] and r2 <= TOL["fp32"]


@pytest.mark.parametrize("chunk,dk,dv", [(16, 128, 128), (32, 64, 64), (128, 128, 128), (64, 16, 16),
                                         (64, 16, 64), (128, 32, 16)])
def test_bf16_general_shapes(chunk, dk, dv):
    x, s0 = make(1, 333, 4, dk, dv, "bf16", seed=7 * chunk + dk, state=True)
    out, st = run(x, "bf16", chunk, s0)
    o64, s64 = oracle.forward(**x, state_in=s0)
    r1, r2 = rel(out, o64), rel(st, s64)
    print(f"C={chunk} dk={dk} dv={dv}: rel-L2 out {r1:.3e} state {r2:.3e}")
    assert r1 <= TOL["bf16"] and r2 <= TOL["bf16"]


@pytest.mark.parametrize("chunk", [32, 128])
def test_fp32_strong_decay_and_resets(chunk):
    x, s0 = make(1, 260, 2, 64, 64, "fp32", seed=5, a_mean=2.0, state=True)
    x["decay"][:, [0, 31, 32, 100, 259]] = 0.0
    out, st = run(x, "fp32", chunk, s0)
    o64, s64 = oracle.forward(**x, state_in=s0)
    assert rel(out, o64) <= TOL["fp32"] and rel(st, s64) <= TOL["fp32"], (rel(out, o64), rel(st, s64))


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_zero_write_is_exact_zero(io):
    x, _ = make(1, 77, 2, 32, 32, io, seed=9)
    x["beta"].zero_()
    out, st = run(x, io, 16)
    assert bool((out == 0).all()) and bool((st == 0).all())


def test_streaming_aligned_split_bit_identical():
    """Calls whose lengths (all but the last) are multiples of chunk_len place the
    chunk grid where one call would: the results are bit-identical."""
    x, s0 = make(1, 250, 3, 64, 32, "fp32", seed=11, state=True)
    d = dev(x)
    g = gb.GDN(1, 3, 64, 32, "fp32", max_T=250)
    o1, st1 = g.forward(d["q"], d["k"], d["v"], d["beta"], d["decay"], state_in=s0.cuda(), chunk_len=32)
    state = s0.cuda().clone()
    outs = []
    for a_, b_ in [(0, 96), (96, 160), (160, 250)]:
        s = slice_tokens(d, a_, b_)
        o, _ = g.forward(s["q"], s["k"], s["v"], s["beta"], s["decay"], state_in=state, state_out=state,
                         chunk_len=32)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=1), o1) and torch.equal(state, st1)
    o64, s64 = oracle.forward(**x, state_in=s0)
    assert rel(o1, o64) <= TOL["fp32"] and rel(st1, s64) <= TOL["fp32"]
    g.close()


@pytest.mark.parametrize("io,chunk", [("fp32", 32), ("bf16", 128)])
def test_bidi_general_and_symmetry(io, chunk):
    x, _ = make(2, 157, 2, 32, 64, io, seed=13)
    d = dev(x)
    g = gb.GDN(2, 2, 32, 64, io, max_T=157, bidi=True)
    out = g.forward_bidi(d["q"], d["k"], d["v"], d["beta"], d["decay"], chunk_len=chunk)
    ob = oracle.bidi(**x)
    assert rel(out, ob) <= TOL[io], rel(out, ob)
    r = reverse_tokens(d)
    out_r = g.forward_bidi(r["q"], r["k"], r["v"], r["beta"], r["decay"], chunk_len=chunk)
    torch.cuda.synchronize()
    assert torch.equal(torch.flip(out_r, dims=[1]), out)
    g.close()


def test_unsupported_chunk_lengths_rejected():
    g = gb.GDN(1, 1, 64, 64, "fp32", max_T=10)
    x = dev(inputs.make_inputs(1, 10, 1, 64, 64, "fp32"))
    out = torch.full((1, 10, 1, 64), 7.0, device="cuda")
    for chunk in (2, 8, 48, 256, -1):
        st = gb.gdn_forward(g.h, x["q"], x["k"], x["v"], x["beta"], x["decay"], None, None, out, 10, chunk,
                            gb.current_stream())
        assert st == gb.GDN_ERR_UNSUPPORTED, chunk
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    g.close()
