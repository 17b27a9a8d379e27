"""The C ABI without a GPU: the library loads, exports every symbol include/gdn.h
declares, and validates arguments on dry-run handles (device = -1), which check
everything and launch nothing.  Pointers here are fake, well-separated addresses;
a dry-run handle never dereferences them."""
import ctypes
import os
import re

import pytest

from gated_deltanet_recurrence_gdn_amd import binding as gb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    with open(os.path.join(ROOT, "include", "gdn.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) >= {"gdn_create", "gdn_forward", "gdn_forward_bidi", "gdn_forward_packed",
                          "gdn_forward_bidi_packed", "gdn_free", "gdn_last_error", "gdn_version"}
    lib = ctypes.CDLL(gb.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in gdn.h but not exported"


def test_version():
    assert re.fullmatch(r"\d+\.\d+\.\d+", gb.gdn_version())


# Fake device addresses: 1 GiB apart, 256-byte aligned.
BASE = 1 << 40
GiB = 1 << 30
ADDR = {n: BASE + i * GiB for i, n in enumerate(["q", "k", "v", "beta", "decay", "s_in", "s_out", "out"])}


@pytest.fixture
def dry():
    st, h = gb.gdn_create(-1, 2, 3, 64, 32, gb.GDN_BF16, 1000, gb.GDN_FLAG_BIDI)
    assert st == gb.GDN_OK and h
    yield h
    gb.gdn_free(h)


def fwd(h, T=100, chunk=1, **over):
    a = dict(ADDR)
    a.update(over)
    return gb.gdn_forward(h, a["q"], a["k"], a["v"], a["beta"], a["decay"], a["s_in"], a["s_out"],
                          a["out"], T, chunk)


def test_dry_run_valid_calls(dry):
    assert fwd(dry) == gb.GDN_OK
    assert fwd(dry, s_in=None, s_out=None) == gb.GDN_OK
    assert fwd(dry, s_out=ADDR["s_in"]) == gb.GDN_OK  # in-place carry
    assert fwd(dry, T=1000) == gb.GDN_OK
    for chunk in (0, 1, 16, 32, 64, 128):
        assert fwd(dry, chunk=chunk) == gb.GDN_OK
    assert fwd(dry, T=0, q=None, k=None, v=None, beta=None, decay=None, out=None) == gb.GDN_OK
    assert gb.gdn_last_error(dry) == ""


@pytest.mark.parametrize("over,code", [
    (dict(T=1001), gb.GDN_ERR_ARG),
    (dict(T=-1), gb.GDN_ERR_ARG),
    (dict(q=None), gb.GDN_ERR_ARG),
    (dict(out=None), gb.GDN_ERR_ARG),
    (dict(decay=None), gb.GDN_ERR_ARG),
    (dict(chunk=7), gb.GDN_ERR_UNSUPPORTED),
    (dict(chunk=-1), gb.GDN_ERR_UNSUPPORTED),
    (dict(chunk=8), gb.GDN_ERR_UNSUPPORTED),
    (dict(chunk=48), gb.GDN_ERR_UNSUPPORTED),
    (dict(chunk=256), gb.GDN_ERR_UNSUPPORTED),
    (dict(q=ADDR["q"] + 8), gb.GDN_ERR_ALIGN),
    (dict(out=ADDR["out"] + 2), gb.GDN_ERR_ALIGN),
    (dict(beta=ADDR["beta"] + 2), gb.GDN_ERR_ALIGN),
    (dict(s_in=ADDR["s_in"] + 4), gb.GDN_ERR_ALIGN),
    (dict(out=ADDR["q"]), gb.GDN_ERR_ALIAS),
    (dict(out=ADDR["v"] + 4096), gb.GDN_ERR_ALIAS),
    (dict(s_out=ADDR["s_in"] + 64), gb.GDN_ERR_ALIAS),
    (dict(s_out=ADDR["out"] + 256), gb.GDN_ERR_ALIAS),
    (dict(s_out=ADDR["k"]), gb.GDN_ERR_ALIAS),
])
def test_dry_run_rejections(dry, over, code):
    assert fwd(dry, **over) == code
    assert gb.gdn_last_error(dry) != ""


def test_beta_unaligned_to_16_is_accepted(dry):
    # gates only need 4-byte alignment (a streaming call can start at any token)
    assert fwd(dry, beta=ADDR["beta"] + 4, decay=ADDR["decay"] + 12) == gb.GDN_OK


def test_alias_edges(dry):
    # out ends exactly where q begins: adjacent, not overlapping
    out_bytes = 2 * 100 * 3 * 32 * 2
    assert fwd(dry, out=ADDR["q"] - out_bytes) == gb.GDN_OK
    assert fwd(dry, out=ADDR["q"] - out_bytes + 16) == gb.GDN_ERR_ALIAS


def test_bidi_dry_run(dry):
    a = ADDR
    assert gb.gdn_forward_bidi(dry, a["q"], a["k"], a["v"], a["beta"], a["decay"], a["out"], 100, 1) == gb.GDN_OK
    assert gb.gdn_forward_bidi(dry, a["q"], a["k"], a["v"], a["beta"], a["decay"], a["q"], 100, 1) == gb.GDN_ERR_ALIAS
    st, h = gb.gdn_create(-1, 1, 1, 16, 16, gb.GDN_F32, 10, 0)
    assert gb.gdn_forward_bidi(h, a["q"], a["k"], a["v"], a["beta"], a["decay"], a["out"], 5, 1) == gb.GDN_ERR_ARG
    assert "GDN_FLAG_BIDI" in gb.gdn_last_error(h)
    gb.gdn_free(h)


# Packed prologue calls on the dry-run handle (B=2, H=3, d_k=64, d_v=32, bf16): the
# packed row is 2 H d_k + H d_v = 480 elements (960 bytes).
ROW = 2 * 3 * 64 + 3 * 32


def pfwd(h, T=100, chunk=1, ts=ROW, bs=None, **over):
    a = dict(ADDR)
    a.update(over)
    bs = T * ts if bs is None else bs
    return gb.gdn_forward_packed(h, a["q"], ts, bs, a["beta"], a["decay"], a["s_in"], a["s_out"], a["out"], T,
                                 chunk)


def test_packed_dry_run_valid_calls(dry):
    assert pfwd(dry) == gb.GDN_OK
    for chunk in (0, 1, 16, 32, 64, 128):
        assert pfwd(dry, chunk=chunk) == gb.GDN_OK
    assert pfwd(dry, ts=ROW + 8) == gb.GDN_OK           # padded rows (976 bytes)
    assert pfwd(dry, bs=0) == gb.GDN_OK                 # both batch elements read the same tokens
    assert pfwd(dry, s_in=None, s_out=None) == gb.GDN_OK
    assert pfwd(dry, s_out=ADDR["s_in"]) == gb.GDN_OK   # in-place carry
    assert pfwd(dry, T=0, q=None, beta=None, decay=None, out=None) == gb.GDN_OK
    assert gb.gdn_last_error(dry) == ""


@pytest.mark.parametrize("over,code", [
    (dict(ts=ROW - 8), gb.GDN_ERR_ARG),
    (dict(ts=ROW + 2), gb.GDN_ERR_ALIGN),
    (dict(bs=-ROW), gb.GDN_ERR_ARG),
    (dict(bs=4), gb.GDN_ERR_ALIGN),
    (dict(ts=(1 << 24) + 8), gb.GDN_ERR_UNSUPPORTED),
    (dict(q=ADDR["q"] + 8), gb.GDN_ERR_ALIGN),
    (dict(out=ADDR["out"] + 8), gb.GDN_ERR_ALIGN),
    (dict(beta=ADDR["beta"] + 2), gb.GDN_ERR_ALIGN),
    (dict(q=None), gb.GDN_ERR_ARG),
    (dict(decay=None), gb.GDN_ERR_ARG),
    (dict(T=1001), gb.GDN_ERR_ARG),
    (dict(chunk=48), gb.GDN_ERR_UNSUPPORTED),
    (dict(out=ADDR["q"] + 4096), gb.GDN_ERR_ALIAS),
    (dict(s_out=ADDR["q"]), gb.GDN_ERR_ALIAS),
    (dict(out=ADDR["beta"]), gb.GDN_ERR_ALIAS),
])
def test_packed_dry_run_rejections(dry, over, code):
    assert pfwd(dry, **over) == code
    assert gb.gdn_last_error(dry) != ""


def test_packed_alias_extent(dry):
    # the extent of qkv is ((B-1) bs + (T-1) ts + row) elements; out may start right after it
    T = 100
    ext = ((2 - 1) * T * ROW + (T - 1) * ROW + ROW) * 2
    assert pfwd(dry, T=T, out=ADDR["q"] + ext) == gb.GDN_OK
    assert pfwd(dry, T=T, out=ADDR["q"] + ext - 16) == gb.GDN_ERR_ALIAS
    # an output in the padding between packed rows still counts as overlapping
    assert pfwd(dry, T=T, ts=ROW + 64, out=ADDR["q"] + 2 * ROW) == gb.GDN_ERR_ALIAS


def test_packed_bidi_dry_run(dry):
    a = ADDR
    ok = gb.gdn_forward_bidi_packed(dry, a["q"], ROW, 100 * ROW, a["beta"], a["decay"], a["out"], 100, 64)
    assert ok == gb.GDN_OK
    bad = gb.gdn_forward_bidi_packed(dry, a["q"], ROW, 100 * ROW, a["beta"], a["decay"], a["q"] + 64, 100, 64)
    assert bad == gb.GDN_ERR_ALIAS
    st, h = gb.gdn_create(-1, 1, 1, 16, 16, gb.GDN_F32, 10, 0)
    assert gb.gdn_forward_bidi_packed(h, a["q"], 48, 480, a["beta"], a["decay"], a["out"], 5, 1) == gb.GDN_ERR_ARG
    assert "GDN_FLAG_BIDI" in gb.gdn_last_error(h)
    gb.gdn_free(h)


def test_torch_wrapper_checks_given_outputs_and_states():
    """out and the states reach the C ABI as raw pointers, so their shapes are checked
    in the wrapper: a state or out of the wrong shape, dtype or layout is refused."""
    import torch
    g = gb.GDN(1, 2, 32, 16, "fp32", max_T=10, device=-1, bidi=True)
    x, v = torch.zeros(1, 4, 2, 32), torch.zeros(1, 4, 2, 16)
    gates = torch.zeros(1, 4, 2)
    for kw in ({"state_in": torch.zeros(1, 2, 32, 16)},          # d_k x d_v instead of d_v x d_k
               {"state_out": torch.zeros(1, 2, 16, 32, dtype=torch.float64)},
               {"state_in": torch.zeros(1, 2, 32, 16).transpose(2, 3)},  # right shape, not contiguous
               {"out": torch.zeros(1, 4, 2, 32)},
               {"out": torch.zeros(1, 4, 2, 16, dtype=torch.bfloat16)}):
        with pytest.raises(ValueError):
            g.forward(x, x, v, gates, gates, **kw)
    with pytest.raises(ValueError):
        g.forward_bidi(x, x, v, gates, gates, out=torch.zeros(1, 3, 2, 16))
    qkv = torch.zeros(1, 4, 2 * 2 * 32 + 2 * 16)
    with pytest.raises(ValueError):
        g.forward_packed(qkv, gates, gates, state_in=torch.zeros(2, 16, 32))
    with pytest.raises(ValueError):
        g.forward_bidi_packed(qkv, gates, gates, out=torch.zeros(1, 4, 2, 17))
    g.close()


def test_torch_wrapper_checks_packed_shapes():
    import torch
    g = gb.GDN(1, 2, 16, 16, "fp32", max_T=10, device=-1)
    with pytest.raises(ValueError):  # W below 2 H d_k + H d_v = 96
        g.forward_packed(torch.zeros(1, 4, 80), torch.zeros(1, 4, 2), torch.zeros(1, 4, 2))
    with pytest.raises(ValueError):  # last stride not 1
        g.forward_packed(torch.zeros(1, 96, 4).transpose(1, 2), torch.zeros(1, 4, 2), torch.zeros(1, 4, 2))
    g.close()


def test_fp8_dry_run_sizes():
    """FP8 inputs are 1 byte, out is bf16: the aliasing extents follow."""
    st, h = gb.gdn_create(-1, 1, 2, 64, 64, gb.GDN_FP8, 100, 0)
    assert st == gb.GDN_OK
    T = 100
    in_bytes = T * 2 * 64        # q, k or v
    out_bytes = T * 2 * 64 * 2   # bf16
    a = dict(ADDR)
    ok = gb.gdn_forward(h, a["q"], a["k"], a["v"], a["beta"], a["decay"], None, None, a["q"] + in_bytes, T, 64)
    assert ok == gb.GDN_OK
    bad = gb.gdn_forward(h, a["q"], a["k"], a["v"], a["beta"], a["decay"], None, None, a["q"] + in_bytes - 16, T, 64)
    assert bad == gb.GDN_ERR_ALIAS
    # out ends exactly where k begins
    ok = gb.gdn_forward(h, a["q"], a["k"], a["v"], a["beta"], a["decay"], None, None, a["k"] - out_bytes, T, 64)
    assert ok == gb.GDN_OK
    # packed rows: strides are multiples of 16 bytes = 16 FP8 elements
    row = 2 * 2 * 64 + 2 * 64
    assert gb.gdn_forward_packed(h, a["q"], row + 16, 0, a["beta"], a["decay"], None, None, a["out"], T, 1) == gb.GDN_OK
    assert gb.gdn_forward_packed(h, a["q"], row + 8, 0, a["beta"], a["decay"], None, None, a["out"], T, 1) == \
        gb.GDN_ERR_ALIGN
    for chunk in (0, 1, 16, 32, 64, 128):
        assert gb.gdn_forward(h, a["q"], a["k"], a["v"], a["beta"], a["decay"], None, None, a["out"], T,
                              chunk) == gb.GDN_OK
    gb.gdn_free(h)


@pytest.mark.parametrize("args,code", [
    ((-1, 0, 1, 16, 16, gb.GDN_F32, 10, 0), gb.GDN_ERR_ARG),
    ((-1, 1, 0, 16, 16, gb.GDN_F32, 10, 0), gb.GDN_ERR_ARG),
    ((-1, 32768, 1, 16, 16, gb.GDN_F32, 10, 0), gb.GDN_ERR_UNSUPPORTED),
    ((-1, 1, 1, 24, 16, gb.GDN_F32, 10, 0), gb.GDN_ERR_UNSUPPORTED),
    ((-1, 1, 1, 16, 256, gb.GDN_F32, 10, 0), gb.GDN_ERR_UNSUPPORTED),
    ((-1, 1, 1, 16, 16, 7, 10, 0), gb.GDN_ERR_UNSUPPORTED),
    ((-1, 1, 1, 16, 16, gb.GDN_F32, -1, 0), gb.GDN_ERR_ARG),
    ((-1, 1, 1, 16, 16, gb.GDN_F32, 10, 8), gb.GDN_ERR_ARG),
    ((-2, 1, 1, 16, 16, gb.GDN_F32, 10, 0), gb.GDN_ERR_ARG),
])
def test_create_rejections(args, code, capfd):
    st, h = gb.gdn_create(*args)
    assert st == code and h is None
    assert gb.gdn_last_error(None) != ""
    assert "gdn_create failed" in capfd.readouterr().err


def test_create_null_args():
    lib = gb.library()
    assert lib.gdn_create(None, None) == gb.GDN_ERR_ARG
    cfg = gb.gdn_config(-1, 1, 1, 16, 16, 0, 1, 0)
    assert lib.gdn_create(ctypes.byref(cfg), None) == gb.GDN_ERR_ARG


def test_free_null_and_null_handle_calls():
    gb.gdn_free(None)
    assert isinstance(gb.gdn_last_error(None), str)
    assert gb.gdn_forward(None, 0, 0, 0, 0, 0, None, None, 0, 0, 1) == gb.GDN_ERR_ARG


def test_create_without_gpu_is_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, h = gb.gdn_create(0, 1, 1, 16, 16, gb.GDN_F32, 10, 0)
    assert st == gb.GDN_ERR_DEVICE and h is None


def test_torch_wrapper_checks_shapes():
    import torch
    g = gb.GDN(1, 2, 16, 16, "fp32", max_T=10, device=-1)
    x = torch.zeros(1, 4, 2, 16)
    with pytest.raises(ValueError):
        g.forward(x, x, x, torch.zeros(1, 4, 3), torch.zeros(1, 4, 2), out=x, state_out=None,
                  return_state=False)
    g.close()


def noalloc(T=100, chunk=64, B=2, H=3, dk=64, dv=32, io=gb.GDN_BF16, flags=0, device=-1, **over):
    cfg = gb.gdn_config(device, B, H, dk, dv, io, 0, flags)
    a = dict(ADDR)
    a.update(over)
    return gb.gdn_forward_noalloc(cfg, a["q"], a["k"], a["v"], a["beta"], a["decay"], a["s_in"], a["s_out"],
                                  a["out"], T, chunk)


def test_noalloc_dry_run():
    """gdn_forward_noalloc validates like gdn_forward (dry run: device = -1) and refuses
    a request whose MFMA-kernel scratch exceeds the fixed array before anything else."""
    assert noalloc() == gb.GDN_OK
    assert noalloc(s_in=None, s_out=None, chunk=1) == gb.GDN_OK
    assert noalloc(s_out=ADDR["s_in"]) == gb.GDN_OK
    assert noalloc(T=0, q=None, k=None, v=None, beta=None, decay=None, out=None) == gb.GDN_OK
    assert noalloc(chunk=3) == gb.GDN_ERR_UNSUPPORTED
    assert noalloc(flags=gb.GDN_FLAG_BIDI) == gb.GDN_ERR_ARG
    assert noalloc(out=ADDR["q"]) == gb.GDN_ERR_ALIAS
    assert noalloc(q=ADDR["q"] + 2) == gb.GDN_ERR_ALIGN
    assert noalloc(T=-1) == gb.GDN_ERR_ARG
    assert noalloc(dk=48) == gb.GDN_ERR_UNSUPPORTED
    assert gb.gdn_last_error(None) != ""
    # capacity: B * H * ceil(T / 64) <= 10,922 chunks (64 MiB of 6 KiB records) on the MFMA kernel
    assert noalloc(B=1, H=20, dk=128, dv=128, T=34944) == gb.GDN_OK
    assert noalloc(B=1, H=20, dk=128, dv=128, T=34945) == gb.GDN_ERR_UNSUPPORTED
    assert "scratch" in gb.gdn_last_error(None)
    # the paths that use no scratch have no such limit
    assert noalloc(B=1, H=20, dk=128, dv=128, T=100000, chunk=1) == gb.GDN_OK
    assert noalloc(B=1, H=20, dk=128, dv=128, T=100000, chunk=32) == gb.GDN_OK
    assert noalloc(B=1, H=20, dk=128, dv=128, T=100000, chunk=64, io=gb.GDN_F32) == gb.GDN_OK
    assert gb.library().gdn_forward_noalloc(None, None, None, None, None, None, None, None, None, 0, 1,
                                            None) == gb.GDN_ERR_ARG


def test_flags_checked():
    """GDN_FLAG_SEGMENTS is a known flag (also with GDN_FLAG_BIDI); any other bit is
    refused at create, and the allocation-free entry point takes no flags."""
    for flags in (gb.GDN_FLAG_SEGMENTS, gb.GDN_FLAG_SEGMENTS | gb.GDN_FLAG_BIDI):
        st, h = gb.gdn_create(-1, 1, 4, 128, 128, gb.GDN_BF16, 5000, flags)
        assert st == gb.GDN_OK, gb.gdn_last_error(None)
        gb.gdn_free(h)
    st, h = gb.gdn_create(-1, 1, 4, 128, 128, gb.GDN_BF16, 5000, 4)
    assert st == gb.GDN_ERR_ARG and "flags" in gb.gdn_last_error(None)
    assert noalloc(flags=gb.GDN_FLAG_SEGMENTS) == gb.GDN_ERR_ARG
