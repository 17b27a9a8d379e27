"""CPU oracle for the Gated-Delta-Net recurrence (ctypes binding of gdn_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package's smoke check
and by the benchmark's CPU-baseline leg, never by the product path.  It shares
no code with the HIP library.

The recurrence, per (batch, head):  S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T,
o_t = S_t q_t / sqrt(d_k).  See gdn_oracle.c for the citations and the forms.

Arrays use the device library's layouts: q, k [B,T,H,d_k]; v, out [B,T,H,d_v];
beta, decay [B,T,H]; state [B,H,d_v,d_k].  Inputs of any real dtype are widened
exactly to float64 (bf16 -> fp32 -> f64 is exact), so the oracle sees the very
values the GPU receives.

The fused input prologue (``unpack_qkv``, ``l2_normalize``, ``sigmoid``,
``decay_from_logit``, ``prologue``, ``forward_packed``, ``bidi_packed``) is plain
numpy float64: split the packed [B, T, 2 H d_k + H d_v] projection into q, k, v
(the column order of the [N, 3C] qkv that the librediffusion PR #21 page's review
splits on the GPU, suggestion "k_split_qkv"), divide q and k by max(||.||_2, 1e-12)
and map the gate logits through b = sigmoid(x_b), a = exp(-softplus(x_a)), then
run the float64 recurrence above.  The pages print neither the normalisation nor
the activations; they are the reading the library documents for the prologue.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c99"]


def build(src: str = _SRC, dst: str = _LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (plain C, no fast-math).  Returns dst."""
    cmd = ["gcc", *CFLAGS, *extra_flags, src, "-o", dst + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(dst + ".tmp", dst)
    return dst


def _stale() -> bool:
    return (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)


def load(path: str | None = None):
    """Load (building first if missing or older than the source) the oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if _stale():
                build()
            _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    L = ctypes.c_long
    lib.oracle_forward_f64.argtypes = [I, L, I, I, I, P, P, P, P, P, P, P, P]
    lib.oracle_forward_f32.argtypes = [I, L, I, I, I, P, P, P, P, P, P, P, P]
    lib.oracle_bidi_f64.argtypes = [I, L, I, I, I, P, P, P, P, P, P]
    lib.oracle_chunkwise_f64.argtypes = [I, L, I, I, I, I, P, P, P, P, P, P, P, P]
    lib.oracle_dense_f64.argtypes = [I, L, I, I, I, P, P, P, P, P, P, P, P]
    lib.oracle_num_threads.restype = I
    for f in ("oracle_forward_f64", "oracle_forward_f32", "oracle_bidi_f64",
              "oracle_chunkwise_f64", "oracle_dense_f64"):
        getattr(lib, f).restype = None
    return lib


def _as(x, dtype):
    """numpy or torch (CPU) array -> contiguous numpy array of dtype (exact widening)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        import torch
        x = x.detach().to("cpu")
        if x.dtype in (torch.bfloat16, torch.float16, torch.float8_e4m3fn, torch.float8_e5m2):
            x = x.float()  # exact: every value of these types is an fp32
        x = x.numpy()
    return np.ascontiguousarray(np.asarray(x), dtype=dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _shapes(q, k, v, beta, decay, state_in):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, T, H, dk), k.shape
    assert v.shape == (B, T, H, dv), v.shape
    assert beta.shape == (B, T, H) and decay.shape == (B, T, H)
    if state_in is not None:
        assert state_in.shape == (B, H, dv, dk), state_in.shape
    return B, T, H, dk, dv


def forward(q, k, v, beta, decay, state_in=None, lib=None):
    """Sequential float64 recurrence.  Returns (out [B,T,H,d_v], state_out [B,H,d_v,d_k])."""
    lib = lib or load()
    q, k, v, beta, decay, s0 = (_as(a, np.float64) for a in (q, k, v, beta, decay, state_in))
    B, T, H, dk, dv = _shapes(q, k, v, beta, decay, s0)
    out = np.zeros((B, T, H, dv), np.float64)
    st = np.zeros((B, H, dv, dk), np.float64)
    lib.oracle_forward_f64(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(decay),
                           _ptr(s0), _ptr(out), _ptr(st))
    return out, st


def forward_f32(q, k, v, beta, decay, state_in=None, lib=None):
    """The same sequential loop in float32 (error-floor reference only)."""
    lib = lib or load()
    q, k, v, beta, decay, s0 = (_as(a, np.float32) for a in (q, k, v, beta, decay, state_in))
    B, T, H, dk, dv = _shapes(q, k, v, beta, decay, s0)
    out = np.zeros((B, T, H, dv), np.float32)
    st = np.zeros((B, H, dv, dk), np.float32)
    lib.oracle_forward_f32(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(decay),
                           _ptr(s0), _ptr(out), _ptr(st))
    return out, st


def bidi(q, k, v, beta, decay, lib=None):
    """fwd(x; 0) + R(fwd(R x; 0)), float64.  Returns out [B,T,H,d_v]."""
    lib = lib or load()
    q, k, v, beta, decay = (_as(a, np.float64) for a in (q, k, v, beta, decay))
    B, T, H, dk, dv = _shapes(q, k, v, beta, decay, None)
    out = np.zeros((B, T, H, dv), np.float64)
    lib.oracle_bidi_f64(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(decay), _ptr(out))
    return out


def chunkwise(q, k, v, beta, decay, state_in=None, chunk=64, lib=None):
    """Chunked (UT-transform) form in float64.  Returns (out, state_out)."""
    lib = lib or load()
    q, k, v, beta, decay, s0 = (_as(a, np.float64) for a in (q, k, v, beta, decay, state_in))
    B, T, H, dk, dv = _shapes(q, k, v, beta, decay, s0)
    out = np.zeros((B, T, H, dv), np.float64)
    st = np.zeros((B, H, dv, dk), np.float64)
    lib.oracle_chunkwise_f64(B, T, H, dk, dv, int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                             _ptr(decay), _ptr(s0), _ptr(out), _ptr(st))
    return out, st


def dense(q, k, v, beta, decay, state_in=None, lib=None):
    """Tiny brute force from explicit transition-matrix products.  T <= 32, d <= 16."""
    lib = lib or load()
    q, k, v, beta, decay, s0 = (_as(a, np.float64) for a in (q, k, v, beta, decay, state_in))
    B, T, H, dk, dv = _shapes(q, k, v, beta, decay, s0)
    assert T <= 64 and dk <= 32, "dense brute force is for tiny inputs only"
    out = np.zeros((B, T, H, dv), np.float64)
    st = np.zeros((B, H, dv, dk), np.float64)
    lib.oracle_dense_f64(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(decay),
                         _ptr(s0), _ptr(out), _ptr(st))
    return out, st


# ---- fused input prologue ------------------------------------------------------

def unpack_qkv(qkv, H: int, dk: int, dv: int):
    """Split a packed [B, T, W] projection (W >= 2 H d_k + H d_v) into float64
    q, k [B,T,H,d_k] and v [B,T,H,d_v]: q of head h at columns h d_k .. h d_k + d_k - 1,
    k after all of q, v after all of k.  Columns past 2 H d_k + H d_v are ignored."""
    x = _as(qkv, np.float64)
    B, T, W = x.shape
    assert W >= 2 * H * dk + H * dv, (W, H, dk, dv)
    q = x[:, :, :H * dk].reshape(B, T, H, dk)
    k = x[:, :, H * dk:2 * H * dk].reshape(B, T, H, dk)
    v = x[:, :, 2 * H * dk:2 * H * dk + H * dv].reshape(B, T, H, dv)
    return np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v)


def l2_normalize(x, eps: float = 1e-12):
    """x / max(||x||_2, eps) over the last axis, float64 (a zero row stays zero)."""
    x = _as(x, np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def sigmoid(x):
    """1 / (1 + e^-x) in float64, evaluated without overflow for either sign."""
    x = _as(x, np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def decay_from_logit(x):
    """exp(-softplus(x)) = exp(-log(1 + e^x)) in float64."""
    x = _as(x, np.float64)
    return np.exp(-np.logaddexp(0.0, x))


def prologue(qkv, beta_logit, decay_logit, H: int, dk: int, dv: int) -> dict:
    """The recurrence inputs the prologue defines: dict(q, k, v, beta, decay), float64."""
    q, k, v = unpack_qkv(qkv, H, dk, dv)
    return dict(q=l2_normalize(q), k=l2_normalize(k), v=v, beta=sigmoid(beta_logit),
                decay=decay_from_logit(decay_logit))


def forward_packed(qkv, beta_logit, decay_logit, H: int, dk: int, dv: int, state_in=None, lib=None):
    """Causal recurrence on the prologue's inputs.  Returns (out, state_out)."""
    return forward(**prologue(qkv, beta_logit, decay_logit, H, dk, dv), state_in=state_in, lib=lib)


def bidi_packed(qkv, beta_logit, decay_logit, H: int, dk: int, dv: int, lib=None):
    """Bidirectional form on the prologue's inputs.  Returns out."""
    return bidi(**prologue(qkv, beta_logit, decay_logit, H, dk, dv), lib=lib)


def num_threads(lib=None) -> int:
    return int((lib or load()).oracle_num_threads())


def rel_l2(x, y) -> float:
    """||x - y||_2 / ||y||_2 over the whole tensor (y is the reference).  If ||y|| = 0
    the result is ||x|| (so exact zeros are required to get 0)."""
    x = _as(x, np.float64).ravel()
    y = _as(y, np.float64).ravel()
    ny = float(np.linalg.norm(y))
    d = float(np.linalg.norm(x - y))
    return d / ny if ny > 0 else d
