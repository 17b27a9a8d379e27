"""Thin ctypes binding of libgdn.so (include/gdn.h), same names as the C ABI.

Argument marshalling only: every step of the recurrence runs in the library's HIP
kernels.  PyTorch is used for device memory and streams.  If libgdn.so is missing
the import of this module raises: there is no fallback implementation.

Raw functions (``gdn_create``, ``gdn_forward``, ``gdn_forward_bidi``,
``gdn_forward_packed``, ``gdn_forward_bidi_packed``, ``gdn_forward_noalloc``, ``gdn_free``,
``gdn_last_error``, ``gdn_version``) take device pointers as ints or torch tensors and return the C
status.  ``GDN`` wraps a handle for torch callers.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgdn.so")

GDN_OK = 0
GDN_ERR_ARG = -1
GDN_ERR_UNSUPPORTED = -2
GDN_ERR_ALIGN = -3
GDN_ERR_ALIAS = -4
GDN_ERR_DEVICE = -5
GDN_ERR_OOM = -6
GDN_ERR_LAUNCH = -7
STATUS_NAMES = {0: "GDN_OK", -1: "GDN_ERR_ARG", -2: "GDN_ERR_UNSUPPORTED", -3: "GDN_ERR_ALIGN",
                -4: "GDN_ERR_ALIAS", -5: "GDN_ERR_DEVICE", -6: "GDN_ERR_OOM", -7: "GDN_ERR_LAUNCH"}
GDN_F32 = 0
GDN_BF16 = 1
GDN_FP8 = 2
GDN_FLAG_BIDI = 1
GDN_FLAG_SEGMENTS = 2


class gdn_config(ctypes.Structure):
    _fields_ = [("device", ctypes.c_int), ("B", ctypes.c_int), ("H", ctypes.c_int),
                ("d_k", ctypes.c_int), ("d_v", ctypes.c_int), ("io_dtype", ctypes.c_int),
                ("max_T", ctypes.c_longlong), ("flags", ctypes.c_uint)]


class GDNError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _load():
    # PyTorch ships its own HIP runtime whose soname (libamdhip64.so.7) is the one
    # libgdn.so needs.  Loading torch first makes the dynamic loader reuse that
    # runtime for libgdn.so, so the process holds one HIP runtime, not two.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m gated_deltanet_recurrence_gdn_amd.build` "
            "(there is no non-HIP implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, LL = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
    lib.gdn_create.argtypes = [ctypes.POINTER(gdn_config), ctypes.POINTER(ctypes.c_void_p)]
    lib.gdn_create.restype = I
    lib.gdn_forward.argtypes = [P, P, P, P, P, P, P, P, P, LL, I, P]
    lib.gdn_forward.restype = I
    lib.gdn_forward_bidi.argtypes = [P, P, P, P, P, P, P, LL, I, P]
    lib.gdn_forward_bidi.restype = I
    lib.gdn_forward_packed.argtypes = [P, P, LL, LL, P, P, P, P, P, LL, I, P]
    lib.gdn_forward_packed.restype = I
    lib.gdn_forward_bidi_packed.argtypes = [P, P, LL, LL, P, P, P, LL, I, P]
    lib.gdn_forward_bidi_packed.restype = I
    lib.gdn_forward_noalloc.argtypes = [ctypes.POINTER(gdn_config), P, P, P, P, P, P, P, P, LL, I, P]
    lib.gdn_forward_noalloc.restype = I
    lib.gdn_free.argtypes = [P]
    lib.gdn_free.restype = None
    lib.gdn_last_error.argtypes = [P]
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_version.argtypes = []
    lib.gdn_version.restype = ctypes.c_char_p
    return lib


_lib = _load()


def library():
    return _lib


def _p(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def gdn_version() -> str:
    return _lib.gdn_version().decode()


def gdn_last_error(h) -> str:
    return _lib.gdn_last_error(h).decode()


def gdn_create(device: int, B: int, H: int, d_k: int, d_v: int, io_dtype: int, max_T: int,
               flags: int = 0):
    """Returns (status, handle); handle is None on failure."""
    cfg = gdn_config(device, B, H, d_k, d_v, io_dtype, max_T, flags)
    h = ctypes.c_void_p()
    st = _lib.gdn_create(ctypes.byref(cfg), ctypes.byref(h))
    return st, (h.value if st == GDN_OK else None)


def gdn_free(h) -> None:
    _lib.gdn_free(h)


def gdn_forward(h, q, k, v, beta, decay, state_in, state_out, out, T: int, chunk_len: int,
                stream=None) -> int:
    return _lib.gdn_forward(h, _p(q), _p(k), _p(v), _p(beta), _p(decay), _p(state_in),
                            _p(state_out), _p(out), int(T), int(chunk_len), stream)


def gdn_forward_bidi(h, q, k, v, beta, decay, out, T: int, chunk_len: int, stream=None) -> int:
    return _lib.gdn_forward_bidi(h, _p(q), _p(k), _p(v), _p(beta), _p(decay), _p(out), int(T),
                                 int(chunk_len), stream)


def gdn_forward_packed(h, qkv, token_stride: int, batch_stride: int, beta_logit, decay_logit, state_in,
                       state_out, out, T: int, chunk_len: int, stream=None) -> int:
    return _lib.gdn_forward_packed(h, _p(qkv), int(token_stride), int(batch_stride), _p(beta_logit),
                                   _p(decay_logit), _p(state_in), _p(state_out), _p(out), int(T),
                                   int(chunk_len), stream)


def gdn_forward_bidi_packed(h, qkv, token_stride: int, batch_stride: int, beta_logit, decay_logit, out,
                            T: int, chunk_len: int, stream=None) -> int:
    return _lib.gdn_forward_bidi_packed(h, _p(qkv), int(token_stride), int(batch_stride), _p(beta_logit),
                                        _p(decay_logit), _p(out), int(T), int(chunk_len), stream)


def gdn_forward_noalloc(cfg: gdn_config, q, k, v, beta, decay, state_in, state_out, out, T: int,
                        chunk_len: int, stream=None) -> int:
    """No handle, no allocation: cfg (a gdn_config) comes with every call; errors are
    read with gdn_last_error(None)."""
    return _lib.gdn_forward_noalloc(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(beta), _p(decay), _p(state_in),
                                    _p(state_out), _p(out), int(T), int(chunk_len), stream)


def current_stream():
    """The raw hipStream_t of torch's current stream on the current device."""
    import torch
    return torch.cuda.current_stream().cuda_stream


class GDN:
    """A handle bound to one (device, B, H, d_k, d_v, dtype, max_T) shape, for torch callers.

    ``forward`` / ``forward_bidi`` check shapes and dtypes on the host, allocate the
    outputs that were not passed in (torch.empty on the same device) and call the C ABI
    on torch's current stream.  Errors raise ``GDNError`` with the library's message.
    """

    def __init__(self, B, H, d_k, d_v, dtype="bf16", max_T=0, device=0, bidi=False, segments=False):
        self.B, self.H, self.d_k, self.d_v = B, H, d_k, d_v
        self.dtype = dtype
        self.io = {"bf16": GDN_BF16, "fp32": GDN_F32, "fp8": GDN_FP8}[dtype]
        self.max_T = max_T
        self.device = device
        self.h = None
        self._free = _lib.gdn_free  # kept on the object: usable while the interpreter shuts down
        flags = (GDN_FLAG_BIDI if bidi else 0) | (GDN_FLAG_SEGMENTS if segments else 0)
        st, h = gdn_create(device, B, H, d_k, d_v, self.io, max_T, flags)
        if st != GDN_OK:
            raise GDNError(st, gdn_last_error(None))
        self.h = h

    def close(self):
        if getattr(self, "h", None) is not None:
            self._free(self.h)
            self.h = None

    __del__ = close

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _check(self, st):
        if st != GDN_OK:
            raise GDNError(st, gdn_last_error(self.h))

    def _torch_dtype(self):
        """dtype of q, k, v (and qkv)."""
        import torch
        return {"bf16": torch.bfloat16, "fp32": torch.float32, "fp8": torch.float8_e4m3fn}[self.dtype]

    def _out_dtype(self):
        """dtype of out: fp32 for fp32 inputs, bf16 otherwise."""
        import torch
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    def _check_inputs(self, q, k, v, beta, decay):
        import torch
        B, H, dk, dv = self.B, self.H, self.d_k, self.d_v
        T = q.shape[1]
        dt = self._torch_dtype()
        for name, x, shape, want in (("q", q, (B, T, H, dk), dt), ("k", k, (B, T, H, dk), dt),
                                     ("v", v, (B, T, H, dv), dt),
                                     ("beta", beta, (B, T, H), torch.float32),
                                     ("decay", decay, (B, T, H), torch.float32)):
            if tuple(x.shape) != shape or x.dtype != want or not x.is_contiguous():
                raise ValueError(f"{name}: expected contiguous {want} {shape}, got {x.dtype} {tuple(x.shape)}")
        return T

    def _check_given(self, T, out=None, state_in=None, state_out=None):
        """Shape, dtype and layout of the caller's out and states.  The C ABI takes raw
        pointers and cannot know their extents, so a wrong shape is refused here."""
        import torch
        st = (self.B, self.H, self.d_v, self.d_k)
        for name, x, shape, want in (("out", out, (self.B, T, self.H, self.d_v), self._out_dtype()),
                                     ("state_in", state_in, st, torch.float32),
                                     ("state_out", state_out, st, torch.float32)):
            if x is not None and (tuple(x.shape) != shape or x.dtype != want or not x.is_contiguous()):
                raise ValueError(f"{name}: expected contiguous {want} {shape}, got {x.dtype} {tuple(x.shape)}")

    def forward(self, q, k, v, beta, decay, state_in=None, state_out=None, out=None,
                chunk_len=64, return_state=True):
        """Causal recurrence.  Returns (out, state_out)."""
        import torch
        T = self._check_inputs(q, k, v, beta, decay)
        self._check_given(T, out, state_in, state_out)
        if out is None:
            out = torch.empty((self.B, T, self.H, self.d_v), dtype=self._out_dtype(), device=q.device)
        if state_out is None and return_state:
            state_out = torch.empty((self.B, self.H, self.d_v, self.d_k), dtype=torch.float32,
                                    device=q.device)
        self._check(gdn_forward(self.h, q, k, v, beta, decay, state_in, state_out, out, T, chunk_len,
                                current_stream()))
        return out, state_out

    def forward_bidi(self, q, k, v, beta, decay, out=None, chunk_len=64):
        """Bidirectional form.  Returns out."""
        import torch
        T = self._check_inputs(q, k, v, beta, decay)
        self._check_given(T, out)
        if out is None:
            out = torch.empty((self.B, T, self.H, self.d_v), dtype=self._out_dtype(), device=q.device)
        self._check(gdn_forward_bidi(self.h, q, k, v, beta, decay, out, T, chunk_len, current_stream()))
        return out

    def _check_packed(self, qkv, beta_logit, decay_logit):
        """qkv: a [B, T, W] tensor (any strides whose last one is 1, W >= 2 H d_k + H d_v)."""
        import torch
        B, H = self.B, self.H
        if qkv.dim() != 3 or qkv.shape[0] != B or qkv.dtype != self._torch_dtype() or qkv.stride(2) != 1:
            raise ValueError(f"qkv: expected a [B={B}, T, W] {self._torch_dtype()} view with unit last stride, "
                             f"got {qkv.dtype} {tuple(qkv.shape)} strides {qkv.stride()}")
        if qkv.shape[2] < 2 * H * self.d_k + H * self.d_v:
            raise ValueError(f"qkv: last dim {qkv.shape[2]} < 2 H d_k + H d_v")
        T = qkv.shape[1]
        for name, x in (("beta_logit", beta_logit), ("decay_logit", decay_logit)):
            if tuple(x.shape) != (B, T, H) or x.dtype != torch.float32 or not x.is_contiguous():
                raise ValueError(f"{name}: expected contiguous float32 {(B, T, H)}, got {x.dtype} {tuple(x.shape)}")
        return T, qkv.stride(1), qkv.stride(0)

    def forward_packed(self, qkv, beta_logit, decay_logit, state_in=None, state_out=None, out=None,
                       chunk_len=64, return_state=True):
        """Causal recurrence with the fused prologue from a packed [B, T, W] qkv view
        (q, k, v of every head side by side in W; L2-normalised q, k and
        sigmoid / exp(-softplus) gates applied in the kernels).  Returns (out, state_out)."""
        import torch
        T, ts, bs = self._check_packed(qkv, beta_logit, decay_logit)
        self._check_given(T, out, state_in, state_out)
        if out is None:
            out = torch.empty((self.B, T, self.H, self.d_v), dtype=self._out_dtype(), device=qkv.device)
        if state_out is None and return_state:
            state_out = torch.empty((self.B, self.H, self.d_v, self.d_k), dtype=torch.float32,
                                    device=qkv.device)
        self._check(gdn_forward_packed(self.h, qkv, ts, bs, beta_logit, decay_logit, state_in, state_out, out, T,
                                       chunk_len, current_stream()))
        return out, state_out

    def forward_bidi_packed(self, qkv, beta_logit, decay_logit, out=None, chunk_len=64):
        """Bidirectional form with the fused prologue.  Returns out."""
        import torch
        T, ts, bs = self._check_packed(qkv, beta_logit, decay_logit)
        self._check_given(T, out)
        if out is None:
            out = torch.empty((self.B, T, self.H, self.d_v), dtype=self._out_dtype(), device=qkv.device)
        self._check(gdn_forward_bidi_packed(self.h, qkv, ts, bs, beta_logit, decay_logit, out, T, chunk_len,
                                            current_stream()))
        return out
