"""Out-of-range writes: out and state_out are placed between two guard regions
filled with a sentinel bit pattern, on every kernel path (MFMA chunked, fp32
chunked, scan, bidirectional, packed prologue), with ragged lengths so that the
last token's row ends exactly at the guard.  The guards must come back intact and
the guarded call must give the bits of an unguarded one.  (The packed-input tests
pad the inputs with NaN, which catches out-of-range reads.)"""
import pytest
import torch

from gated_deltanet_recurrence_gdn_amd import inputs
from gated_deltanet_recurrence_gdn_amd import binding as gb
from gpu_util import dev

pytestmark = pytest.mark.gpu

G = 4096            # guard elements on each side (a multiple of 16 bytes for every dtype)
SENTINEL = 0x7FC3   # a NaN bit pattern in bf16; as int32 0x7FC37FC3, also a NaN in fp32


def guarded(shape, dtype):
    """(buffer, view): view is a contiguous tensor of `shape` with G sentinel elements
    on each side inside buffer."""
    n = 1
    for s in shape:
        n *= s
    buf = torch.empty(n + 2 * G, dtype=dtype, device="cuda")
    raw = buf.view(torch.int16) if dtype.itemsize == 2 else buf.view(torch.int32)
    raw.fill_(SENTINEL if dtype.itemsize == 2 else (SENTINEL << 16) | SENTINEL)
    return buf, buf[G:G + n].view(shape)


def guards_intact(buf, n):
    raw = buf.view(torch.int16) if buf.element_size() == 2 else buf.view(torch.int32)
    want = SENTINEL if buf.element_size() == 2 else (SENTINEL << 16) | SENTINEL
    return bool((raw[:G] == want).all()) and bool((raw[G + n:] == want).all())


CASES = [  # (io, d_k, d_v, chunk, T)
    ("bf16", 128, 128, 64, 137), ("bf16", 64, 32, 64, 100), ("fp8", 128, 64, 64, 71),
    ("fp32", 64, 64, 32, 77), ("bf16", 32, 16, 16, 45), ("bf16", 128, 128, 1, 50), ("fp32", 16, 64, 1, 33)]


@pytest.mark.parametrize("io,dk,dv,chunk,T", CASES, ids=lambda v: str(v))
def test_causal_writes_stay_in_bounds(io, dk, dv, chunk, T):
    B, H = 2, 3
    x = dev(inputs.make_inputs(B, T, H, dk, dv, io, seed=dk + dv + T))
    s0 = 0.3 * torch.randn((B, H, dv, dk), device="cuda", generator=torch.Generator("cuda").manual_seed(3))
    g = gb.GDN(B, H, dk, dv, io, max_T=T)
    odt = torch.float32 if io == "fp32" else torch.bfloat16
    ob, out = guarded((B, T, H, dv), odt)
    sb, st = guarded((B, H, dv, dk), torch.float32)
    g.forward(x["q"], x["k"], x["v"], x["beta"], x["decay"], state_in=s0, state_out=st, out=out, chunk_len=chunk)
    ref_out, ref_st = g.forward(x["q"], x["k"], x["v"], x["beta"], x["decay"], state_in=s0, chunk_len=chunk)
    torch.cuda.synchronize()
    g.close()
    assert guards_intact(ob, out.numel()), "out guard overwritten"
    assert guards_intact(sb, st.numel()), "state_out guard overwritten"
    assert torch.equal(out.view(torch.int16) if odt == torch.bfloat16 else out.view(torch.int32),
                       ref_out.view(torch.int16) if odt == torch.bfloat16 else ref_out.view(torch.int32))
    assert torch.equal(st, ref_st)


@pytest.mark.parametrize("io,d,chunk,T", [("bf16", 128, 64, 129), ("bf16", 64, 1, 70), ("fp32", 32, 16, 50)],
                         ids=lambda v: str(v))
def test_bidi_writes_stay_in_bounds(io, d, chunk, T):
    B, H = 1, 5
    x = dev(inputs.make_inputs(B, T, H, d, d, io, seed=d + T))
    g = gb.GDN(B, H, d, d, io, max_T=T, bidi=True)
    odt = torch.float32 if io == "fp32" else torch.bfloat16
    ob, out = guarded((B, T, H, d), odt)
    g.forward_bidi(x["q"], x["k"], x["v"], x["beta"], x["decay"], out=out, chunk_len=chunk)
    ref = g.forward_bidi(x["q"], x["k"], x["v"], x["beta"], x["decay"], chunk_len=chunk)
    torch.cuda.synchronize()
    g.close()
    assert guards_intact(ob, out.numel())
    assert torch.equal(out.float().nan_to_num(7.0), ref.float().nan_to_num(7.0))


def test_packed_writes_stay_in_bounds():
    B, T, H, d = 2, 99, 4, 128
    xp = inputs.make_packed_inputs(B, T, H, d, d, "bf16", seed=5, pad=16, gap=2)
    buf = xp["qkv_buf"].cuda()
    qkv = buf[:, :T, :xp["qkv"].shape[2]]
    bl, dl = xp["beta_logit"].cuda(), xp["decay_logit"].cuda()
    g = gb.GDN(B, H, d, d, "bf16", max_T=T)
    ob, out = guarded((B, T, H, d), torch.bfloat16)
    sb, st = guarded((B, H, d, d), torch.float32)
    g.forward_packed(qkv, bl, dl, state_out=st, out=out, chunk_len=64)
    ref_out, ref_st = g.forward_packed(qkv, bl, dl, chunk_len=64)
    torch.cuda.synchronize()
    g.close()
    assert guards_intact(ob, out.numel()) and guards_intact(sb, st.numel())
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)) and torch.equal(st, ref_st)
