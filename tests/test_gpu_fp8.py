"""Parity of FP8 (OCP E4M3) q, k, v inputs with the float64 oracle, through the C ABI:
the bf16 MFMA chunked kernel, the fp32 general kernel, the scan, the bidirectional
form and the fused prologue.  The oracle reads the FP8 values exactly, so the bar is
the bf16 one (the kernels widen FP8 to bf16 / fp32 exactly and then compute as for
bf16 inputs); out is bf16."""
import pytest
import torch

import oracle
from gated_deltanet_recurrence_gdn_amd import inputs
from gated_deltanet_recurrence_gdn_amd import binding as gb
from gpu_util import parity_by_head, TOL, dev, host, rel, reverse_tokens, slice_tokens

pytestmark = pytest.mark.gpu


def make(B, T, H, dk, dv, seed=0, a_mean=0.0, state=False):
    x = inputs.make_inputs(B, T, H, dk, dv, "fp8", seed=seed, a_mean=a_mean)
    s0 = None
    if state:
        g = torch.Generator().manual_seed(seed + 5000)
        s0 = 0.3 * torch.randn((B, H, dv, dk), generator=g, dtype=torch.float32)
    return x, s0


def run(x, s0=None, chunk=64):
    B, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    g = gb.GDN(B, H, dk, dv, "fp8", max_T=T)
    d = dev(x)
    out, st = g.forward(d["q"], d["k"], d["v"], d["beta"], d["decay"],
                        state_in=None if s0 is None else s0.cuda(), chunk_len=chunk)
    torch.cuda.synchronize()
    g.close()
    assert out.dtype == torch.bfloat16
    return out, st


def check(out, st, x, s0, what):
    o64, s64 = oracle.forward(**x, state_in=s0)
    r1, r2 = rel(out, o64), rel(st, s64)
    print(f"{what}: rel-L2 out {r1:.3e} state {r2:.3e}")
    assert r1 <= TOL["fp8"] and r2 <= TOL["fp8"], (r1, r2)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (32, 128), (128, 32)])
def test_mfma_dims_ragged_with_state(dk, dv):
    x, s0 = make(2, 150, 3, dk, dv, seed=dk + 2 * dv, state=True)
    out, st = run(x, s0)
    check(out, st, x, s0, f"mfma dk={dk} dv={dv}")


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_mfma_lengths(T):
    x, s0 = make(1, T, 8, 64, 64, seed=T, state=True)
    out, st = run(x, s0)
    check(out, st, x, s0, f"mfma T={T}")


@pytest.mark.parametrize("chunk,dk,dv", [(1, 128, 128), (1, 64, 32), (1, 16, 16), (32, 64, 64), (16, 16, 64),
                                         (128, 32, 16)])
def test_scan_and_general(chunk, dk, dv):
    x, s0 = make(2, 133, 3, dk, dv, seed=chunk + dk + dv, state=True)
    out, st = run(x, s0, chunk)
    check(out, st, x, s0, f"C={chunk} dk={dk} dv={dv}")


def test_extreme_codes():
    """The largest (+-448) and subnormal (2^-9 .. 7 * 2^-9) E4M3 values in v and k,
    strong decay: still within the bar, no overflow."""
    x, s0 = make(1, 200, 2, 64, 64, seed=31, a_mean=2.0, state=True)
    g = torch.Generator().manual_seed(8)
    for name, vals in (("v", [448.0, -448.0, 2.0 ** -9, -7 * 2.0 ** -9]), ("k", [2.0 ** -9, 3 * 2.0 ** -9])):
        t = x[name].float()
        idx = torch.randint(0, t.numel(), (300,), generator=g)
        t.view(-1)[idx] = torch.tensor(vals).repeat(300 // len(vals))
        x[name] = t.to(torch.float8_e4m3fn)
    for chunk in (64, 1):
        out, st = run(x, s0, chunk)
        assert bool(torch.isfinite(out.float()).all())
        check(out, st, x, s0, f"extreme codes C={chunk}")


@pytest.mark.parametrize("chunk", [64, 1])
def test_bidi_and_reversal(chunk):
    x, _ = make(1, 190, 2, 64, 64, seed=3 + chunk)
    d = dev(x)
    g = gb.GDN(1, 2, 64, 64, "fp8", max_T=190, bidi=True)
    out = g.forward_bidi(d["q"], d["k"], d["v"], d["beta"], d["decay"], chunk_len=chunk)
    r = reverse_tokens(d)
    out_r = g.forward_bidi(r["q"], r["k"], r["v"], r["beta"], r["decay"], chunk_len=chunk)
    torch.cuda.synchronize()
    g.close()
    assert torch.equal(torch.flip(out_r, dims=[1]), out)
    ob = oracle.bidi(**x)
    assert rel(out, ob) <= TOL["fp8"], rel(out, ob)


@pytest.mark.parametrize("chunk", [1, 64])
def test_streaming_split_bit_identical(chunk):
    x, s0 = make(1, 320, 4, 128, 128, seed=44, state=True)
    d = dev(x)
    g = gb.GDN(1, 4, 128, 128, "fp8", max_T=320)
    o1, st1 = g.forward(d["q"], d["k"], d["v"], d["beta"], d["decay"], state_in=s0.cuda(), chunk_len=chunk)
    state = s0.cuda().clone()
    outs = []
    for a_, b_ in [(0, 128), (128, 192), (192, 320)]:
        s = slice_tokens(d, a_, b_)
        o, _ = g.forward(s["q"], s["k"], s["v"], s["beta"], s["decay"], state_in=state, state_out=state,
                         chunk_len=chunk)
        outs.append(o)
    torch.cuda.synchronize()
    g.close()
    assert torch.equal(torch.cat(outs, dim=1), o1) and torch.equal(state, st1)


@pytest.mark.parametrize("chunk,d", [(64, 128), (64, 64), (64, 32), (1, 128)])
def test_packed_prologue(chunk, d):
    """FP8 packed projection with the fused prologue (normalisation of the FP8 q, k
    in the kernels), padded token stride and a gap between batch elements."""
    B, T, H = 2, 170, 3
    x = inputs.make_packed_inputs(B, T, H, d, d, "fp8", seed=12 + d, pad=32, gap=3)
    g0 = torch.Generator().manual_seed(77)
    s0 = 0.3 * torch.randn((B, H, d, d), generator=g0, dtype=torch.float32)
    buf = x["qkv_buf"].cuda()
    qkv = buf[:, :T, :x["qkv"].shape[2]]
    g = gb.GDN(B, H, d, d, "fp8", max_T=T)
    out, st = g.forward_packed(qkv, x["beta_logit"].cuda(), x["decay_logit"].cuda(), state_in=s0.cuda(),
                               chunk_len=chunk)
    torch.cuda.synchronize()
    g.close()
    o64, s64 = oracle.forward_packed(x["qkv"], x["beta_logit"], x["decay_logit"], H, d, d, state_in=s0)
    r1, r2 = oracle.rel_l2(host(out), o64), oracle.rel_l2(host(st), s64)
    print(f"packed fp8 C={chunk} d={d}: rel-L2 out {r1:.3e} state {r2:.3e}")
    assert r1 <= TOL["fp8"] and r2 <= TOL["fp8"]


def test_full_size_all_heads():
    """The bench shape (B=2, H=32, T=32760, d=128, decay exp(-softplus(N(2,1)))) with
    FP8 q, k, v on the MFMA path: every head vs the oracle, per head and per edge chunk."""
    w = inputs.WORKLOADS["batched_bf16_d128"]
    x = inputs.make_inputs(w.B, w.T, w.H, w.dk, w.dv, "fp8", seed=0, a_mean=w.a_mean)
    d = dev(x)
    g = gb.GDN(w.B, w.H, w.dk, w.dv, "fp8", max_T=w.T)
    out, st = g.forward(d["q"], d["k"], d["v"], d["beta"], d["decay"], chunk_len=64)
    torch.cuda.synchronize()
    g.close()
    del d
    assert bool(torch.isfinite(out.float()).all())
    o64, s64 = oracle.forward(**x)
    parity_by_head("fp8 full size", out, o64, TOL["fp8"], st, s64)


@pytest.mark.parametrize("chunk", [64, 1])
@pytest.mark.parametrize("which", ["q", "k", "v"])
def test_every_code_widens_exactly(which, chunk):
    """All 256 E4M3 codes through the library, bit-exact.  With a_t = 0 every token
    starts from S = 0, so o_t = v_t (k_t . q_t) / sqrt(d_k) exactly.  Token t carries
    code t at one place of `which`, the other two are unit vectors picking it out
    (q_t = k_t = e_{t mod 32} for q and k, v_t = e_0), so o_t[0] is the code's value
    times fp32(1/sqrt(32)), rounded once to bf16.  The two NaN codes go through q
    only (o_t = NaN); in k or v a NaN enters the state and, since 0 * NaN is NaN,
    every later output of any exact evaluation, so there they are replaced by 0."""
    T, d = 256, 32
    f8 = torch.float8_e4m3fn
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(f8).float()  # NaN stays NaN
    if which != "q":
        codes = torch.nan_to_num(codes, nan=0.0)
    q = torch.zeros(1, T, 1, d)
    k = torch.zeros(1, T, 1, d)
    v = torch.zeros(1, T, 1, d)
    t = torch.arange(T)
    q[0, t, 0, t % d] = 1.0
    k[0, t, 0, t % d] = 1.0
    v[0, t, 0, 0] = 1.0
    if which == "v":
        v[0, t, 0, 0] = codes
    else:
        {"q": q, "k": k}[which][0, t, 0, t % d] = codes
    x = {"q": q.to(f8), "k": k.to(f8), "v": v.to(f8), "beta": torch.ones(1, T, 1), "decay": torch.zeros(1, T, 1)}
    out, _ = run(x, None, chunk)
    got = out[0, :, 0, 0].float().cpu()
    scale = torch.tensor(1.0 / 32 ** 0.5, dtype=torch.float32)
    want = (codes * scale).to(torch.bfloat16).float()
    nan = torch.isnan(codes)
    assert bool(torch.isnan(got[nan]).all())
    assert torch.equal(got[~nan], want[~nan])
