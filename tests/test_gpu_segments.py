"""The segment-parallel causal form (GDN_FLAG_SEGMENTS) against the float64 oracle.

A call on a handle with the flag is cut into token segments that run concurrently
(segment 0 from state_in, the others from zero and from the identity), then combined;
the recurrence being affine in the state makes the result the same up to rounding.
Every head, its first and final partial chunk, and the final state are compared with
the oracle at the bf16 bar.  A segmented call must also differ in its low bits from
the one-sweep call of the same inputs (else it did not run segmented)."""
import pytest
import torch

import oracle
from gated_deltanet_recurrence_gdn_amd import inputs
from gated_deltanet_recurrence_gdn_amd import binding as gb
from gpu_util import TOL, dev, parity_by_head, slice_tokens

pytestmark = pytest.mark.gpu


def state0(B, H, dv, dk, seed, scale=0.3):
    g = torch.Generator().manual_seed(seed)
    return scale * torch.randn((B, H, dv, dk), generator=g, dtype=torch.float32)


def run(x, s0, segments, io="bf16", chunk=64, max_T=None):
    B, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    g = gb.GDN(B, H, dk, dv, io, max_T=max_T or T, segments=segments)
    d = dev(x)
    out, st = g.forward(d["q"], d["k"], d["v"], d["beta"], d["decay"],
                        state_in=None if s0 is None else s0.cuda(), chunk_len=chunk)
    torch.cuda.synchronize()
    g.close()
    return out, st


def check(label, x, s0, io="bf16"):
    out, st = run(x, s0, True, io)
    ref, _ = run(x, s0, False, io)
    print(f"[gpu case] {label}", flush=True)
    assert not torch.equal(out, ref), f"{label}: the call did not run segmented"
    o64, s64 = oracle.forward(**x, state_in=s0)
    parity_by_head(label, out, o64, TOL[io], st, s64)


def test_d64_workload_segmented():
    """B=1, H=16, T=4680, d=64: 32 blocks per sweep, so four segments fit."""
    x = inputs.make_workload("causal_bf16_d64")
    check("3 frames d=64, segments", x, None)


@pytest.mark.parametrize("dk,dv,T,H", [(128, 128, 4680, 20), (128, 128, 1500, 4), (64, 128, 2000, 6),
                                       (128, 32, 1100, 8), (32, 64, 3333, 3)])
def test_dims_ragged_with_state(dk, dv, T, H):
    x = inputs.make_inputs(1, T, H, dk, dv, "bf16", seed=dk + dv + T)
    s0 = state0(1, H, dv, dk, seed=T)
    check(f"dk={dk} dv={dv} T={T} H={H}, state_in", x, s0)


@pytest.mark.parametrize("B,H,dk,dv,T", [(2, 4, 128, 128, 3000), (3, 2, 64, 64, 2100)])
def test_batch_with_state(B, H, dk, dv, T):
    """Several batch elements: every (b, h) has its own segment states, transitions and
    start states (4 segments each)."""
    x = inputs.make_inputs(B, T, H, dk, dv, "bf16", seed=100 * B + T)
    s0 = state0(B, H, dv, dk, seed=T + 1)
    check(f"B={B} H={H} dk={dk} dv={dv} T={T}, state_in", x, s0)


def test_no_state_out():
    """state_out NULL: the combine launches no state row (5 segments)."""
    B, H, d, T = 2, 3, 64, 2600
    x = inputs.make_inputs(B, T, H, d, d, "bf16", seed=31)
    s0 = state0(B, H, d, d, seed=32)
    d_ = dev(x)
    outs = {}
    for seg in (True, False):
        g = gb.GDN(B, H, d, d, "bf16", max_T=T, segments=seg)
        o, st = g.forward(d_["q"], d_["k"], d_["v"], d_["beta"], d_["decay"], state_in=s0.cuda(),
                          return_state=False)
        torch.cuda.synchronize()
        g.close()
        assert st is None
        outs[seg] = o
    print("[gpu case] no state_out, segments", flush=True)
    assert not torch.equal(outs[True], outs[False])
    o64, _ = oracle.forward(**x, state_in=s0)
    parity_by_head("no state_out, segments", outs[True], o64, TOL["bf16"])


def test_long_memory_heads():
    """Decay close to 1 (a = exp(-softplus(x)), x ~ N(-2, 1)): the start state reaches
    every later token, so the correction carries most of each output."""
    x = inputs.make_inputs(1, 3000, 4, 128, 128, "bf16", seed=5, a_mean=-2.0)
    s0 = state0(1, 4, 128, 128, seed=6, scale=1.0)
    check("long memory, state_in", x, s0)


def test_fp8_inputs():
    x = inputs.make_inputs(1, 2500, 4, 128, 128, "fp8", seed=7)
    s0 = state0(1, 4, 128, 128, seed=8)
    check("FP8 inputs, state_in", x, s0, io="fp8")


def test_streaming_five_calls():
    """Config 2's split (5 calls of 4,680 tokens, H = 20, d = 128) with the state
    carried between calls, in place; each call's outputs and the final state against
    one oracle run over all 23,400 tokens."""
    x = inputs.make_workload("streaming_bf16_d128")
    B, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    n = T // 5
    g = gb.GDN(B, H, dk, dv, "bf16", max_T=n, segments=True)
    st = torch.zeros((B, H, dv, dk), device="cuda")
    outs = []
    for c in range(5):
        d = dev(slice_tokens(x, c * n, (c + 1) * n))
        o, _ = g.forward(d["q"], d["k"], d["v"], d["beta"], d["decay"], state_in=st, state_out=st)
        outs.append(o)
    torch.cuda.synchronize()
    g.close()
    o64, s64 = oracle.forward(**x)
    parity_by_head("5 segmented calls", torch.cat(outs, dim=1), o64, TOL["bf16"], st, s64)


def test_packed_prologue():
    B, T, H, d = 1, 2200, 4, 128
    xp = inputs.make_packed_inputs(B, T, H, d, d, "bf16", seed=9, pad=8)
    qkv = xp["qkv_buf"].cuda()[:, :T, :xp["qkv"].shape[2]]
    bl, dl = xp["beta_logit"].cuda(), xp["decay_logit"].cuda()
    outs = {}
    for seg in (True, False):
        g = gb.GDN(B, H, d, d, "bf16", max_T=T, segments=seg)
        outs[seg] = g.forward_packed(qkv, bl, dl)
        torch.cuda.synchronize()
        g.close()
    assert not torch.equal(outs[True][0], outs[False][0])
    o64, s64 = oracle.forward_packed(xp["qkv"], xp["beta_logit"], xp["decay_logit"], H, d, d)
    parity_by_head("packed prologue, segments", outs[True][0], o64, TOL["bf16"], outs[True][1], s64)


def test_short_call_is_one_sweep():
    """Below two segments of 8 chunks the handle runs the plain sweep, bit for bit."""
    x = inputs.make_inputs(1, 900, 4, 128, 128, "bf16", seed=11)
    s0 = state0(1, 4, 128, 128, seed=12)
    a, sa = run(x, s0, True)
    b, sb = run(x, s0, False)
    assert torch.equal(a, b) and torch.equal(sa, sb)


def test_graph_replay():
    """The segmented call (two streams, fork and join by events) captured in a HIP
    graph: every replay equals the eager call bit for bit."""
    x = inputs.make_inputs(1, 2000, 4, 64, 64, "bf16", seed=13)
    d = dev(x)
    g = gb.GDN(1, 4, 64, 64, "bf16", max_T=2000, segments=True)
    s0 = state0(1, 4, 64, 64, seed=14).cuda()
    out = torch.empty((1, 2000, 4, 64), dtype=torch.bfloat16, device="cuda")
    st = torch.empty((1, 4, 64, 64), device="cuda")

    def call(stream):
        assert gb.gdn_forward(g.h, d["q"], d["k"], d["v"], d["beta"], d["decay"], s0, st, out, 2000, 64,
                              stream) == gb.GDN_OK

    call(gb.current_stream())
    torch.cuda.synchronize()
    eager = (out.clone(), st.clone())
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=side):
        call(side.cuda_stream)
    torch.cuda.synchronize()
    for _ in range(3):
        out.zero_()
        st.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[0]) and torch.equal(st, eager[1])
    g.close()


@pytest.mark.parametrize("segments", [False, True])
def test_long_sequence(segments):
    """2^18 + 3 tokens (4,097 chunks, the last of 3 tokens) on two heads at d = 64 with a
    start state: one sweep, and the segmented form (8 segments of 513 chunks)."""
    T = (1 << 18) + 3
    x = inputs.make_inputs(1, T, 2, 64, 64, "bf16", seed=21)
    s0 = state0(1, 2, 64, 64, seed=22)
    if segments:
        check(f"T={T}, segments", x, s0)
        return
    print(f"[gpu case] T={T}, one sweep", flush=True)
    out, st = run(x, s0, False)
    o64, s64 = oracle.forward(**x, state_in=s0)
    parity_by_head(f"T={T}, one sweep", out, o64, TOL["bf16"], st, s64)
