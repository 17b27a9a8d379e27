"""Short sequences on every path (the bf16 MFMA chunked kernel, the fp32 general
chunked kernel and the scan, selected by chunk length and input type).

* T = 0 writes only the state: state_in is copied to state_out exactly (zeros
  without state_in), out is left untouched, and q, k, v and the gates may be NULL.
* The bidirectional form at T = 1, 2, 63, 64, 65 (one partial chunk, one full
  chunk, a full chunk and one token) equals the float64 oracle's sum of the
  forward and the reverse recurrence within the bar."""
import pytest
import torch

import oracle
from gated_deltanet_recurrence_gdn_amd import inputs
from gated_deltanet_recurrence_gdn_amd import binding as gb
from gpu_util import TOL, dev, rel

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("io,chunk,d", [("bf16", 64, 128), ("fp8", 64, 64), ("bf16", 64, 32), ("fp32", 32, 64),
                                        ("bf16", 16, 32), ("fp32", 1, 16)])
def test_zero_tokens_write_only_the_state(io, chunk, d):
    B, H = 2, 3
    g = gb.GDN(B, H, d, d, io, max_T=64)
    s0 = 0.3 * torch.randn((B, H, d, d), device="cuda")
    st = torch.full_like(s0, 5.0)
    sentinel = torch.full((B, 1, H, d), 7.0, device="cuda")
    stream = gb.current_stream()
    assert gb.gdn_forward(g.h, None, None, None, None, None, s0, st, sentinel, 0, chunk, stream) == gb.GDN_OK
    torch.cuda.synchronize()
    assert torch.equal(st, s0) and bool((sentinel == 7.0).all())

    st.fill_(5.0)
    assert gb.gdn_forward(g.h, None, None, None, None, None, None, st, None, 0, chunk, stream) == gb.GDN_OK
    torch.cuda.synchronize()
    assert bool((st == 0).all())

    # the packed entry point, in place (state_in = state_out)
    row = 2 * H * d + H * d
    st.copy_(s0)
    assert gb.gdn_forward_packed(g.h, None, row, 0, None, None, st, st, None, 0, chunk, stream) == gb.GDN_OK
    torch.cuda.synchronize()
    assert torch.equal(st, s0)
    g.close()


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65])
@pytest.mark.parametrize("io,chunk,d", [("bf16", 64, 64), ("fp8", 64, 32), ("fp32", 32, 32), ("fp32", 1, 32)])
def test_bidi_short(io, chunk, d, T):
    B, H = 1, 2
    x = inputs.make_inputs(B, T, H, d, d, io, seed=100 + T)
    dx = dev(x)
    g = gb.GDN(B, H, d, d, io, max_T=T, bidi=True)
    out = g.forward_bidi(dx["q"], dx["k"], dx["v"], dx["beta"], dx["decay"], chunk_len=chunk)
    torch.cuda.synchronize()
    g.close()
    r = rel(out, oracle.bidi(**x))
    print(f"bidi {io} C={chunk} d={d} T={T}: rel-L2 {r:.3e}")
    assert r <= TOL[io]
