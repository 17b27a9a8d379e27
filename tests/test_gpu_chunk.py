"""Parity of the chunked form (chunk_len = 64, bf16 MFMA) with the float64 oracle,
through the C ABI on the GPU."""
import pytest
import torch

import oracle
from gated_deltanet_recurrence_gdn_amd import inputs
from gated_deltanet_recurrence_gdn_amd import binding as gb
from gpu_util import parity_by_head, TOL, dev, rel, reverse_tokens, slice_tokens

pytestmark = pytest.mark.gpu


def make(B, T, H, dk, dv, seed=0, a_mean=0.0, state=False):
    x = inputs.make_inputs(B, T, H, dk, dv, "bf16", seed=seed, a_mean=a_mean)
    s0 = None
    if state:
        g = torch.Generator().manual_seed(seed + 1000)
        s0 = 0.3 * torch.randn((B, H, dv, dk), generator=g, dtype=torch.float32)
    return x, s0


def run(x, s0=None, chunk=64):
    B, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    g = gb.GDN(B, H, dk, dv, "bf16", max_T=T)
    d = dev(x)
    out, st = g.forward(d["q"], d["k"], d["v"], d["beta"], d["decay"],
                        state_in=None if s0 is None else s0.cuda(), chunk_len=chunk)
    torch.cuda.synchronize()
    g.close()
    return out, st


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 64), (128, 128), (128, 32), (32, 128), (64, 128)])
def test_dims_ragged_with_state(dk, dv):
    x, s0 = make(2, 150, 3, dk, dv, seed=dk + 2 * dv, state=True)
    out, st = run(x, s0)
    o64, s64 = oracle.forward(**x, state_in=s0)
    r1, r2 = rel(out, o64), rel(st, s64)
    print(f"dk={dk} dv={dv}: rel-L2 out {r1:.3e} state {r2:.3e}")
    assert r1 <= TOL["bf16"] and r2 <= TOL["bf16"]


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 128, 200])
def test_lengths_xcd_mapped(T):
    # 8 heads: the blocks of one head are placed on one XCD
    x, s0 = make(1, T, 8, 64, 64, seed=T, state=True)
    out, st = run(x, s0)
    o64, s64 = oracle.forward(**x, state_in=s0)
    assert rel(out, o64) <= TOL["bf16"] and rel(st, s64) <= TOL["bf16"], (rel(out, o64), rel(st, s64))


def test_bf16_d64_workload():
    """B=1, H=16, T=4680 (3 frames of 30x52 tokens), d=64, chunk_len=64."""
    x = inputs.make_workload("causal_bf16_d64")
    out, st = run(x)
    o64, s64 = oracle.forward(**x)
    r1, r2 = rel(out, o64), rel(st, s64)
    print(f"rel-L2 out {r1:.3e} state {r2:.3e}")
    assert r1 <= TOL["bf16"] and r2 <= TOL["bf16"]


def test_strong_decay_and_resets():
    x, s0 = make(1, 300, 4, 128, 128, seed=3, a_mean=2.0, state=True)
    x["decay"][:, [0, 64, 65, 130, 299]] = 0.0
    out, st = run(x, s0)
    o64, s64 = oracle.forward(**x, state_in=s0)
    assert rel(out, o64) <= TOL["bf16"] and rel(st, s64) <= TOL["bf16"], (rel(out, o64), rel(st, s64))


def test_zero_write_is_exact_zero():
    x, _ = make(1, 130, 2, 64, 64, seed=4)
    x["beta"].zero_()
    out, st = run(x)
    assert bool((out == 0).all()) and bool((st == 0).all())


def test_streaming_d128():
    """5 calls of 4680 tokens carrying the fp32 state vs one 23400-token call.

    4680 = 73*64 + 8, so the chunk grid of the split run differs from the one-shot
    run: equal within rounding, checked against the oracle.  With every call but the
    last a multiple of 64 tokens (4672 x 4 + 4712) the chunk grids coincide and the
    results are bit-identical."""
    w = inputs.WORKLOADS["streaming_bf16_d128"]
    x = inputs.make_workload(w)
    d = dev(x)
    g = gb.GDN(w.B, w.H, w.dk, w.dv, "bf16", max_T=w.T)
    out1, st1 = g.forward(d["q"], d["k"], d["v"], d["beta"], d["decay"], chunk_len=64)
    o64, s64 = oracle.forward(**x)
    assert rel(out1, o64) <= TOL["bf16"] and rel(st1, s64) <= TOL["bf16"]

    def split_run(cuts):
        state = torch.zeros((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device="cuda")
        outs = []
        for a_, b_ in zip(cuts[:-1], cuts[1:]):
            s = slice_tokens(d, a_, b_)
            o, _ = g.forward(s["q"], s["k"], s["v"], s["beta"], s["decay"], state_in=state,
                             state_out=state, chunk_len=64)
            outs.append(o)
        torch.cuda.synchronize()
        return torch.cat(outs, dim=1), state

    n = w.T // w.calls
    o5, s5 = split_run([i * n for i in range(w.calls + 1)])
    print(f"literal split: rel-L2 vs oracle out {rel(o5, o64):.3e} state {rel(s5, s64):.3e}")
    assert rel(o5, o64) <= TOL["bf16"] and rel(s5, s64) <= TOL["bf16"]
    oa, sa = split_run([0, 4672, 2 * 4672, 3 * 4672, 4 * 4672, w.T])
    assert torch.equal(oa, out1) and torch.equal(sa, st1)
    g.close()


def test_bidi_chunked_and_symmetry():
    x, _ = make(2, 201, 3, 64, 64, seed=12)
    d = dev(x)
    g = gb.GDN(2, 3, 64, 64, "bf16", max_T=201, bidi=True)
    out = g.forward_bidi(d["q"], d["k"], d["v"], d["beta"], d["decay"], chunk_len=64)
    ob = oracle.bidi(**x)
    assert rel(out, ob) <= TOL["bf16"], rel(out, ob)
    r = reverse_tokens(d)
    out_r = g.forward_bidi(r["q"], r["k"], r["v"], r["beta"], r["decay"], chunk_len=64)
    torch.cuda.synchronize()
    assert torch.equal(torch.flip(out_r, dims=[1]), out)
    g.close()


@pytest.mark.parametrize("T", [64, 65, 127, 128, 129, 191, 192, 193, 320, 333, 449, 1920, 1921, 1984, 2049, 2113])
@pytest.mark.parametrize("d", [64, 128])
def test_bidi_split_sweep(T, d):
    """The MFMA kernel's bidirectional form walks chunks [0, n1) of both directions
    (n1 = ceil(n / 2); in two launches split at ceil(n1 / 2) once n1 >= 16, i.e. from
    T = 1921) and [n1, n) in a last one, adding the other direction's first-half
    output; the middle tokens both first halves cover are combined separately.
    Lengths around the split points and the middle overlap, against the oracle per
    head and per edge chunk, plus exact reversal symmetry."""
    B, H = 2, 3
    x, _ = make(B, T, H, d, d, seed=T + d)
    dx = dev(x)
    g = gb.GDN(B, H, d, d, "bf16", max_T=T, bidi=True)
    out = g.forward_bidi(dx["q"], dx["k"], dx["v"], dx["beta"], dx["decay"], chunk_len=64)
    r = reverse_tokens(dx)
    out_r = g.forward_bidi(r["q"], r["k"], r["v"], r["beta"], r["decay"], chunk_len=64)
    torch.cuda.synchronize()
    g.close()
    assert torch.equal(torch.flip(out_r, dims=[1]), out)
    parity_by_head(f"bidi split T={T} d={d}", out, oracle.bidi(**x), TOL["bf16"])


def test_state_in_untouched_and_inplace():
    x, s0 = make(1, 100, 2, 128, 64, seed=21, state=True)
    d = dev(x)
    g = gb.GDN(1, 2, 128, 64, "bf16", max_T=100)
    s_in = s0.cuda()
    keep = s_in.clone()
    o1, st1 = g.forward(d["q"], d["k"], d["v"], d["beta"], d["decay"], state_in=s_in, chunk_len=64)
    torch.cuda.synchronize()
    assert torch.equal(s_in, keep)
    o2, _ = g.forward(d["q"], d["k"], d["v"], d["beta"], d["decay"], state_in=s_in, state_out=s_in,
                      chunk_len=0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s_in, st1)
    g.close()
