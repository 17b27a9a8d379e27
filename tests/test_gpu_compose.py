"""How calls compose: resuming from a state saved to host memory, the
bidirectional form against two causal calls, and separate handles on concurrent
streams.

* A state copied to the host between calls and copied back into a fresh device
  tensor resumes the sequence exactly: the result equals one call bit for bit (the
  scan at any split, the chunked form at chunk-aligned splits).
* gdn_forward_bidi(x) = gdn_forward(x) + R(gdn_forward(R x)), both from zero state:
  bit for bit with fp32 I/O (the bidirectional form's fp32 partials are exactly those
  outputs and their sum is rounded once), within the bf16 bar with bf16 I/O (the two
  causal outputs are rounded before they are added)."""
import pytest
import torch

from gated_deltanet_recurrence_gdn_amd import inputs
from gated_deltanet_recurrence_gdn_amd import binding as gb
from gpu_util import TOL, dev, rel, reverse_tokens, slice_tokens

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("io,chunk,d", [("bf16", 1, 128), ("bf16", 64, 128), ("fp32", 32, 64), ("fp8", 64, 64)])
def test_resume_from_host_saved_state(io, chunk, d):
    B, T, H, split = 1, 256, 3, 128
    x = dev(inputs.make_inputs(B, T, H, d, d, io, seed=61))
    g = gb.GDN(B, H, d, d, io, max_T=T)
    o1, st1 = g.forward(x["q"], x["k"], x["v"], x["beta"], x["decay"], chunk_len=chunk)
    a = slice_tokens(x, 0, split)
    oa, sa = g.forward(a["q"], a["k"], a["v"], a["beta"], a["decay"], chunk_len=chunk)
    saved = sa.cpu()          # the state leaves the device ...
    del sa
    torch.cuda.synchronize()
    resumed = saved.cuda()    # ... and comes back in a fresh allocation
    b = slice_tokens(x, split, T)
    ob, sb = g.forward(b["q"], b["k"], b["v"], b["beta"], b["decay"], state_in=resumed, chunk_len=chunk)
    torch.cuda.synchronize()
    g.close()
    assert torch.equal(torch.cat([oa, ob], dim=1), o1)
    assert torch.equal(sb, st1)


@pytest.mark.parametrize("io,chunk", [("fp32", 1), ("fp32", 32), ("fp32", 64), ("bf16", 64), ("bf16", 1)])
def test_bidi_is_two_causal_calls(io, chunk):
    B, T, H, d = 2, 190, 2, 64
    x = dev(inputs.make_inputs(B, T, H, d, d, io, seed=62))
    g = gb.GDN(B, H, d, d, io, max_T=T, bidi=True)
    ob = g.forward_bidi(x["q"], x["k"], x["v"], x["beta"], x["decay"], chunk_len=chunk)
    of, _ = g.forward(x["q"], x["k"], x["v"], x["beta"], x["decay"], chunk_len=chunk, return_state=False)
    r = reverse_tokens(x)
    orr, _ = g.forward(r["q"], r["k"], r["v"], r["beta"], r["decay"], chunk_len=chunk, return_state=False)
    torch.cuda.synchronize()
    g.close()
    two = of.float() + torch.flip(orr, dims=[1]).float()
    if io == "fp32":
        assert torch.equal(ob, two)
    else:
        r_ = rel(ob, two.double().cpu().numpy())
        print(f"bf16 bidi vs two rounded causal calls: rel-L2 {r_:.3e}")
        assert r_ <= TOL["bf16"]


def test_two_handles_on_two_streams_concurrently():
    """Separate handles share nothing: two chunked calls and two bidi calls enqueued on
    two streams at once give the same bits as the same calls run one after another."""
    B, T, H, d = 1, 640, 4, 128
    xa = dev(inputs.make_inputs(B, T, H, d, d, "bf16", seed=71))
    xb = dev(inputs.make_inputs(B, T, H, d, d, "bf16", seed=72))
    ga = gb.GDN(B, H, d, d, "bf16", max_T=T, bidi=True)
    gbb = gb.GDN(B, H, d, d, "bf16", max_T=T, bidi=True)

    def calls(g, x, stream):
        with torch.cuda.stream(stream):
            o, s = g.forward(x["q"], x["k"], x["v"], x["beta"], x["decay"], chunk_len=64)
            ob = g.forward_bidi(x["q"], x["k"], x["v"], x["beta"], x["decay"], chunk_len=64)
        return o, s, ob

    main = torch.cuda.current_stream()
    ref_a = calls(ga, xa, main)
    ref_b = calls(gbb, xb, main)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(main)
    sb.wait_stream(main)
    got_a = calls(ga, xa, sa)
    got_b = calls(gbb, xb, sb)
    torch.cuda.synchronize()
    ga.close()
    gbb.close()
    for r, g_ in zip(ref_a + ref_b, got_a + got_b):
        assert torch.equal(r, g_)
