"""The forward calls enqueue kernels only (no allocation, synchronisation or host copy),
so a caller can capture them in a HIP graph.  Captured streaming (5 calls carrying the
state in place), chunked and scan forms, bidirectional form and the packed prologue:
every replay, with the program's own eager work and synchronisations between
replays, must equal the eager result bit for bit."""
import pytest
import torch

from gated_deltanet_recurrence_gdn_amd import inputs
from gated_deltanet_recurrence_gdn_amd import binding as gb
from gpu_util import dev

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _replay_and_check(graph, outs, eager, reset):
    for i in range(REPLAYS):
        reset()
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {i} differs from the eager result"
        # eager work of the program between replays
        torch.randn(1024, device="cuda").sum().item()


@pytest.mark.parametrize("chunk", [64, 1])
def test_streaming_calls_in_one_graph(chunk):
    B, H, d, n, calls = 1, 4, 128, 192, 5
    x = dev(inputs.make_inputs(B, n * calls, H, d, d, "bf16", seed=21))
    parts = [{k: v[:, i * n:(i + 1) * n].contiguous() for k, v in x.items()} for i in range(calls)]
    g = gb.GDN(B, H, d, d, "bf16", max_T=n)
    s0 = 0.1 * torch.randn((B, H, d, d), device="cuda")
    state = torch.empty_like(s0)
    outs = [torch.empty((B, n, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(calls)]

    def run(stream):
        for i, pi in enumerate(parts):
            assert gb.gdn_forward(g.h, pi["q"], pi["k"], pi["v"], pi["beta"], pi["decay"], state, state, outs[i], n,
                                  chunk, stream) == gb.GDN_OK

    state.copy_(s0)
    run(gb.current_stream())
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs] + [state.clone()]

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    state.copy_(s0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        run(side.cuda_stream)
    torch.cuda.synchronize()
    _replay_and_check(graph, outs + [state], eager, lambda: state.copy_(s0))
    g.close()


def test_bidi_and_packed_in_one_graph():
    B, T, H, d = 1, 200, 2, 64
    x = dev(inputs.make_inputs(B, T, H, d, d, "bf16", seed=22))
    xp = inputs.make_packed_inputs(B, T, H, d, d, "bf16", seed=23, pad=8)
    qkv = xp["qkv_buf"].cuda()[:, :T, :xp["qkv"].shape[2]]
    bl, dl = xp["beta_logit"].cuda(), xp["decay_logit"].cuda()
    g = gb.GDN(B, H, d, d, "bf16", max_T=T, bidi=True)
    ob = torch.empty((B, T, H, d), dtype=torch.bfloat16, device="cuda")
    op = torch.empty_like(ob)
    st = torch.empty((B, H, d, d), device="cuda")

    def run(stream):
        assert gb.gdn_forward_bidi(g.h, x["q"], x["k"], x["v"], x["beta"], x["decay"], ob, T, 64,
                                   stream) == gb.GDN_OK
        assert gb.gdn_forward_packed(g.h, qkv, qkv.stride(1), qkv.stride(0), bl, dl, None, st, op, T, 64,
                                     stream) == gb.GDN_OK

    run(gb.current_stream())
    torch.cuda.synchronize()
    eager = [ob.clone(), op.clone(), st.clone()]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=side):
        run(side.cuda_stream)
    torch.cuda.synchronize()
    _replay_and_check(graph, [ob, op, st], eager, lambda: None)
    g.close()
