"""The scan launcher switches to 16 state values per lane (scan_kernel<DK, 16, ...>)
once 8 per lane would put more than two waves on every SIMD: at d_k = 128 that is
more than 64 (direction, b, h) rows of heads, at d_k = 64 more than 256 (with
d_v = 64), at d_k = 32 more than 1024 (d_v = 32), at d_k = 16 more than 4096
(d_v = 16).  These cases sit just past each threshold (small T, many heads) and are
checked against the float64 oracle, with and without a carried state, in fp32 at the
fp32 bar and in bf16, plus a bidirectional case and a two-call split that must equal
one call bit for bit."""
import pytest
import torch

import oracle
from gated_deltanet_recurrence_gdn_amd import inputs
from gated_deltanet_recurrence_gdn_amd import binding as gb
from gpu_util import TOL, dev, host, slice_tokens

pytestmark = pytest.mark.gpu

# (B, H, d_k, d_v, T): each just past its E = 16 threshold
WIDE = [(1, 65, 128, 128, 100), (1, 257, 64, 64, 70), (1, 1025, 32, 32, 40), (2, 2049, 16, 16, 30),
        (1, 513, 16, 128, 33)]


def _state(B, H, dv, dk, seed):
    g = torch.Generator().manual_seed(seed)
    return 0.3 * torch.randn((B, H, dv, dk), generator=g, dtype=torch.float32)


@pytest.mark.parametrize("io", ["fp32", "bf16"])
@pytest.mark.parametrize("state", [False, True])
@pytest.mark.parametrize("B,H,dk,dv,T", WIDE, ids=lambda v: str(v))
def test_wide_scan(B, H, dk, dv, T, io, state):
    x = inputs.make_inputs(B, T, H, dk, dv, io, seed=H + dk)
    s0 = _state(B, H, dv, dk, H) if state else None
    d = dev(x)
    g = gb.GDN(B, H, dk, dv, io, max_T=T)
    out, st = g.forward(d["q"], d["k"], d["v"], d["beta"], d["decay"],
                        state_in=None if s0 is None else s0.cuda(), chunk_len=1)
    torch.cuda.synchronize()
    g.close()
    o64, s64 = oracle.forward(**x, state_in=s0)
    r1, r2 = oracle.rel_l2(host(out), o64), oracle.rel_l2(host(st), s64)
    print(f"E=16 scan B={B} H={H} dk={dk} dv={dv} {io} state={state}: rel-L2 out {r1:.3e} state {r2:.3e}")
    assert r1 <= TOL[io] and r2 <= TOL[io]


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_wide_scan_bidi(io):
    """B=2, H=33, d=128: 132 (direction, b, h) rows, past the d_k = 128 threshold."""
    B, H, d, T = 2, 33, 128, 90
    x = inputs.make_inputs(B, T, H, d, d, io, seed=7)
    dx = dev(x)
    g = gb.GDN(B, H, d, d, io, max_T=T, bidi=True)
    out = g.forward_bidi(dx["q"], dx["k"], dx["v"], dx["beta"], dx["decay"], chunk_len=1)
    torch.cuda.synchronize()
    g.close()
    r = oracle.rel_l2(host(out), oracle.bidi(**x))
    print(f"E=16 bidi {io}: rel-L2 {r:.3e}")
    assert r <= TOL[io]


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_wide_scan_split_is_bit_identical(io):
    """Two calls (37 + 63 tokens, state carried) give the bits of one 100-token call."""
    B, H, d, T, t1 = 1, 65, 128, 100, 37
    x = inputs.make_inputs(B, T, H, d, d, io, seed=11)
    s0 = _state(B, H, d, d, 12).cuda()
    dx = dev(x)
    g = gb.GDN(B, H, d, d, io, max_T=T)
    out, st = g.forward(dx["q"], dx["k"], dx["v"], dx["beta"], dx["decay"], state_in=s0, chunk_len=1)
    a, b = dev(slice_tokens(x, 0, t1)), dev(slice_tokens(x, t1, T))
    o1, s1 = g.forward(a["q"], a["k"], a["v"], a["beta"], a["decay"], state_in=s0, chunk_len=1)
    o2, s2 = g.forward(b["q"], b["k"], b["v"], b["beta"], b["decay"], state_in=s1, chunk_len=1)
    torch.cuda.synchronize()
    g.close()
    assert torch.equal(torch.cat([o1, o2], dim=1), out)
    assert torch.equal(s2, st)
