"""gdn_forward_noalloc (no handle, no allocation; the MFMA kernel's scratch is the
library's fixed per-GPU device array) against gdn_forward through the C ABI: two
calls in a row, the second with a smaller input, each bit-identical to gdn_forward
on the same inputs and within the bar of the float64 oracle; the paths that need
no scratch; a request beyond the array's capacity refused before any launch."""
import pytest
import torch

import oracle
from gated_deltanet_recurrence_gdn_amd import inputs
from gated_deltanet_recurrence_gdn_amd import binding as gb
from gpu_util import TOL, dev, host

pytestmark = pytest.mark.gpu

IO = {"bf16": gb.GDN_BF16, "fp32": gb.GDN_F32, "fp8": gb.GDN_FP8}


def run_both(B, H, dk, dv, io, T, chunk, seed, state=True):
    x = inputs.make_inputs(B, T, H, dk, dv, io, seed=seed)
    s0 = None
    if state:
        s0 = 0.3 * torch.randn((B, H, dv, dk), generator=torch.Generator().manual_seed(seed), dtype=torch.float32)
    d = dev(x)
    sd = None if s0 is None else s0.cuda()
    odt = torch.float32 if io == "fp32" else torch.bfloat16
    stream = gb.current_stream()
    # the handle path
    g = gb.GDN(B, H, dk, dv, io, max_T=T)
    ref_out, ref_st = g.forward(d["q"], d["k"], d["v"], d["beta"], d["decay"], state_in=sd, chunk_len=chunk)
    torch.cuda.synchronize()
    g.close()
    # the no-allocation path, outputs pre-filled with NaN
    out = torch.full((B, T, H, dv), float("nan"), dtype=odt, device="cuda")
    st = torch.full((B, H, dv, dk), float("nan"), dtype=torch.float32, device="cuda")
    cfg = gb.gdn_config(0, B, H, dk, dv, IO[io], 0, 0)
    r = gb.gdn_forward_noalloc(cfg, d["q"], d["k"], d["v"], d["beta"], d["decay"], sd, st, out, T, chunk, stream)
    assert r == gb.GDN_OK, gb.gdn_last_error(None)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(st, ref_st), "noalloc differs from gdn_forward"
    o64, s64 = oracle.forward(**x, state_in=s0)
    r1, r2 = oracle.rel_l2(host(out), o64), oracle.rel_l2(host(st), s64)
    print(f"noalloc B={B} H={H} d={dk}/{dv} {io} T={T} C={chunk}: rel-L2 out {r1:.3e} state {r2:.3e}", flush=True)
    assert r1 <= TOL[io] and r2 <= TOL[io]


def test_two_calls_second_smaller():
    # 20 heads x 74 chunks (the 5-call streaming workload's call), then 16 heads at d = 64
    run_both(1, 20, 128, 128, "bf16", 4680, 64, seed=1)
    run_both(1, 16, 64, 64, "bf16", 1000, 64, seed=2)


def test_paths_without_scratch():
    run_both(2, 3, 128, 128, "bf16", 90, 1, seed=3)     # scan
    run_both(1, 4, 64, 32, "fp32", 77, 32, seed=4)      # fp32 chunked kernel
    run_both(1, 2, 64, 64, "fp8", 130, 64, seed=5)      # FP8 on the MFMA kernel


def test_beyond_capacity_is_refused():
    B, H, d, T = 1, 20, 128, 35000   # 20 x 547 chunks > 10,922
    x = dev(inputs.make_inputs(B, 64, H, d, d, "bf16", seed=6))
    q = torch.zeros((B, T, H, d), dtype=torch.bfloat16, device="cuda")
    gates = torch.zeros((B, T, H), dtype=torch.float32, device="cuda")
    out = torch.full((B, T, H, d), 3.0, dtype=torch.bfloat16, device="cuda")
    cfg = gb.gdn_config(0, B, H, d, d, gb.GDN_BF16, 0, 0)
    r = gb.gdn_forward_noalloc(cfg, q, q, q, gates, gates, None, None, out, T, 64, gb.current_stream())
    assert r == gb.GDN_ERR_UNSUPPORTED
    assert "scratch" in gb.gdn_last_error(None)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
    # one chunk less per head is accepted at the boundary: 20 x 546 chunks
    r = gb.gdn_forward_noalloc(cfg, q, q, q, gates, gates, None, None, out, 34944, 64, gb.current_stream())
    assert r == gb.GDN_OK, gb.gdn_last_error(None)
    torch.cuda.synchronize()
    del x
