"""MI355X (gfx950) gated delta-rule mixer: Python binding of libgdr.

The functions here carry the C ABI's names (``include/gdr.h``) and do only
argument marshalling: shapes and dtypes are read from torch tensors, which
provide device memory and the current stream; every step of the computation
runs in the HIP kernels of ``libgdr.so``. There is no fallback: importing
this package without a built ``libgdr.so`` raises.

Tensor layouts (contiguous, on the same GPU):
  prefill  q, k [B,T,Hqk,D]; v [B,T,Hv,D]; beta [B,T,Hv] f32;
           g [B,T,Hv] or [B,T,Hv,D] f32; b [B,T,Hv,D]; w [B,T,Hv,D];
           state [B,Hv,D,D] f32 (row = key channel, column = value channel)
  decode   the same without the T axis.
  recurrent (short runs from a live state) as prefill.
q, k, v, b, w and the output share one dtype: torch.bfloat16 or torch.float32.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdr.so")

GDR_OK, GDR_E_INVAL, GDR_E_UNSUPPORTED, GDR_E_HIP, GDR_E_NOMEM = 0, -1, -2, -3, -4
GDR_F32, GDR_BF16 = 0, 1
GDR_DECAY_NONE, GDR_DECAY_SCALAR, GDR_DECAY_CHANNEL = 0, 1, 2
CHUNK = 64
GDR_NOALLOC_SCRATCH_BYTES = 64 << 20  # the workspace array of gdr_chunk_fwd_noalloc

# Every symbol include/gdr.h declares.
EXPORTS = ("gdr_state_bytes", "gdr_state_alloc", "gdr_state_free", "gdr_chunk_workspace_bytes",
           "gdr_chunk_fwd_in_workspace_bytes",
           "gdr_chunk_fwd", "gdr_decode_step", "gdr_recurrent_fwd", "gdr_recurrent_fwd_in", "gdr_chunk_fwd_in",
           "gdr_recurrent_bwd_workspace_bytes", "gdr_recurrent_bwd", "gdr_chunk_bwd_workspace_bytes", "gdr_chunk_bwd",
           "gdr_chunk_fwd_noalloc", "gdr_norm_la_workspace_bytes", "gdr_norm_la_fwd", "gdr_norm_la_decode_step",
           "gdr_last_error", "gdr_version")


class GdrError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libgdr status {status}: {message}")
        self.status = status


class gdr_input_stage(ctypes.Structure):
    _fields_ = [("conv_w", ctypes.c_void_p), ("conv_in", ctypes.c_void_p), ("conv_out", ctypes.c_void_p),
                ("decay_scale", ctypes.c_void_p)]


class gdr_desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H_qk", ctypes.c_int), ("H_v", ctypes.c_int),
                ("d_k", ctypes.c_int), ("d_v", ctypes.c_int), ("io_dtype", ctypes.c_int),
                ("decay", ctypes.c_int), ("chunk", ctypes.c_int), ("scale", ctypes.c_float)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run gated_delta_rule_23_amd/build.py "
                          "(or __graft_entry__.build()) first; there is no non-HIP fallback")
    # torch ships its own HIP runtime with the same SONAME (libamdhip64.so.7).
    # Loading torch first makes libgdr.so bind to that runtime, so the library
    # and torch share one runtime, one device context and the same streams.
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover - C-only use without torch
        pass
    lib = ctypes.CDLL(LIB_PATH)
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    D = ctypes.POINTER(gdr_desc)
    lib.gdr_state_bytes.restype = S
    lib.gdr_state_bytes.argtypes = [I, I, I, I]
    lib.gdr_state_alloc.restype = I
    lib.gdr_state_alloc.argtypes = [I, I, I, I, ctypes.POINTER(P), ctypes.POINTER(S), P]
    lib.gdr_state_free.restype = I
    lib.gdr_state_free.argtypes = [P]
    lib.gdr_chunk_workspace_bytes.restype = I
    lib.gdr_chunk_workspace_bytes.argtypes = [D, ctypes.POINTER(S)]
    lib.gdr_chunk_fwd_in_workspace_bytes.restype = I
    lib.gdr_chunk_fwd_in_workspace_bytes.argtypes = [D, ctypes.POINTER(S)]
    lib.gdr_chunk_fwd.restype = I
    lib.gdr_chunk_fwd.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, S, P]
    lib.gdr_chunk_fwd_noalloc.restype = I
    lib.gdr_chunk_fwd_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P]
    lib.gdr_norm_la_workspace_bytes.restype = I
    lib.gdr_norm_la_workspace_bytes.argtypes = [D, ctypes.POINTER(S)]
    lib.gdr_norm_la_fwd.restype = I
    lib.gdr_norm_la_fwd.argtypes = [D, P, P, P, P, P, P, P, P, P, S, P]
    lib.gdr_norm_la_decode_step.restype = I
    lib.gdr_norm_la_decode_step.argtypes = [D, P, P, P, P, P, P, P]
    lib.gdr_decode_step.restype = I
    lib.gdr_decode_step.argtypes = [D, P, P, P, P, P, P, P, P, P, P]
    lib.gdr_recurrent_fwd.restype = I
    lib.gdr_recurrent_fwd.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P]
    lib.gdr_recurrent_fwd_in.restype = I
    lib.gdr_recurrent_fwd_in.argtypes = [D, ctypes.POINTER(gdr_input_stage), P, P, P, P, P, P, P, P, P, P, P]
    lib.gdr_chunk_fwd_in.restype = I
    lib.gdr_chunk_fwd_in.argtypes = [D, ctypes.POINTER(gdr_input_stage), P, P, P, P, P, P, P, P, P, P, P, S, P]
    lib.gdr_recurrent_bwd_workspace_bytes.restype = I
    lib.gdr_recurrent_bwd_workspace_bytes.argtypes = [D, ctypes.POINTER(S)]
    lib.gdr_recurrent_bwd.restype = I
    lib.gdr_recurrent_bwd.argtypes = [D] + [P] * 19 + [S, P]
    lib.gdr_chunk_bwd_workspace_bytes.restype = I
    lib.gdr_chunk_bwd_workspace_bytes.argtypes = [D, ctypes.POINTER(S)]
    lib.gdr_chunk_bwd.restype = I
    lib.gdr_chunk_bwd.argtypes = [D] + [P] * 19 + [S, P]
    lib.gdr_last_error.restype = ctypes.c_char_p
    lib.gdr_last_error.argtypes = []
    lib.gdr_version.restype = I
    lib.gdr_version.argtypes = []
    return lib


lib = _load()


def _check(rc: int):
    if rc != GDR_OK:
        raise GdrError(rc, lib.gdr_last_error().decode())


def gdr_last_error() -> str:
    return lib.gdr_last_error().decode()


def gdr_version() -> int:
    return lib.gdr_version()


def gdr_state_bytes(B: int, H_v: int, d_k: int, d_v: int) -> int:
    return lib.gdr_state_bytes(B, H_v, d_k, d_v)


def gdr_state_alloc(B: int, H_v: int, d_k: int, d_v: int, stream=None):
    """Allocate a zero-filled fp32 state through the library. Returns (device
    pointer as int, bytes); free it with gdr_state_free."""
    p, n = ctypes.c_void_p(), ctypes.c_size_t()
    _check(lib.gdr_state_alloc(B, H_v, d_k, d_v, ctypes.byref(p), ctypes.byref(n), _stream(stream)))
    return p.value, n.value


def gdr_state_free(ptr) -> None:
    _check(lib.gdr_state_free(ptr))


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else t.data_ptr()


def _torch_stream(stream, dev):
    """The torch stream a call runs on: the current one, a torch stream, or a
    raw HIP stream handle. Tensors a call allocates are made on it (under
    torch.cuda.stream), so that the caching allocator does not hand their
    memory to another stream while the call's kernels may still use it."""
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream(dev)
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream, device=dev)
    return stream


def _stream(stream):
    if stream is None:
        torch = _torch()
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    return stream if isinstance(stream, int) else stream.cuda_stream


def _io_dtype(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return GDR_BF16
    if t.dtype == torch.float32:
        return GDR_F32
    raise TypeError(f"io tensors must be bfloat16 or float32, got {t.dtype}")


def _require(t, name, shape=None, dtype=None, device=None):
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def make_desc(B, T, Hqk, Hv, D, io, decay, scale=1.0, chunk=CHUNK) -> gdr_desc:
    return gdr_desc(B, T, Hqk, Hv, D, D, io, decay, chunk, float(scale))


def gdr_chunk_workspace_bytes(desc: gdr_desc) -> int:
    n = ctypes.c_size_t()
    _check(lib.gdr_chunk_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def gdr_chunk_fwd_in_workspace_bytes(desc: gdr_desc) -> int:
    n = ctypes.c_size_t()
    _check(lib.gdr_chunk_fwd_in_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def _decay_of(g, lead, Hv, D):
    if g is None:
        return GDR_DECAY_NONE
    if tuple(g.shape) == tuple(lead) + (Hv,):
        return GDR_DECAY_SCALAR
    if tuple(g.shape) == tuple(lead) + (Hv, D):
        return GDR_DECAY_CHANNEL
    raise ValueError(f"g has shape {tuple(g.shape)}")


def gdr_chunk_fwd(q, k, v, *, g=None, beta=None, b=None, w=None, S0=None, scale=1.0, chunk=CHUNK,
                  o=None, ST=None, workspace=None, stream=None):
    """Chunked prefill. Returns (o, ST); ST may be passed equal to S0 for an
    in-place state update. ``workspace`` (a uint8 tensor of at least
    gdr_chunk_workspace_bytes) is allocated here when not given."""
    torch = _torch()
    B, T, Hqk, D = q.shape
    Hv = v.shape[2]
    dev, io_t = q.device, q.dtype
    for name, t, shape in (("q", q, (B, T, Hqk, D)), ("k", k, (B, T, Hqk, D)), ("v", v, (B, T, Hv, D)),
                           ("b", b, (B, T, Hv, D)), ("w", w, (B, T, Hv, D))):
        _require(t, name, shape, io_t, dev)
    _require(beta, "beta", (B, T, Hv), torch.float32, dev)
    _require(g, "g", None, torch.float32, dev)
    _require(S0, "S0", (B, Hv, D, D), torch.float32, dev)
    desc = make_desc(B, T, Hqk, Hv, D, _io_dtype(q), _decay_of(g, (B, T), Hv, D), scale, chunk)
    s = _torch_stream(stream, dev)
    with torch.cuda.stream(s):
        if o is None:
            o = torch.empty((B, T, Hv, D), dtype=io_t, device=dev)
        if ST is None:
            ST = torch.empty((B, Hv, D, D), dtype=torch.float32, device=dev)
        nbytes = gdr_chunk_workspace_bytes(desc)
        if workspace is None and nbytes > 0:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _require(o, "o", (B, T, Hv, D), io_t, dev)
    _require(ST, "ST", (B, Hv, D, D), torch.float32, dev)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.gdr_chunk_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(b),
                             _ptr(w), _ptr(S0), _ptr(o), _ptr(ST), _ptr(workspace), wsz, _stream(s)))
    return o, ST


def gdr_chunk_fwd_noalloc(q, k, v, *, o, ST, g=None, beta=None, b=None, w=None, S0=None, scale=1.0, chunk=CHUNK,
                          stream=None):
    """gdr_chunk_fwd with the library's own device workspace: allocates
    nothing, so the outputs o [B,T,Hv,D] and ST [B,Hv,D,D] are the caller's.
    The call's workspace must fit GDR_NOALLOC_SCRATCH_BYTES; calls that
    overlap in time on one GPU share that workspace and race."""
    torch = _torch()
    B, T, Hqk, D = q.shape
    Hv = v.shape[2]
    dev, io_t = q.device, q.dtype
    for name, t, shape in (("q", q, (B, T, Hqk, D)), ("k", k, (B, T, Hqk, D)), ("v", v, (B, T, Hv, D)),
                           ("b", b, (B, T, Hv, D)), ("w", w, (B, T, Hv, D))):
        _require(t, name, shape, io_t, dev)
    _require(beta, "beta", (B, T, Hv), torch.float32, dev)
    _require(g, "g", None, torch.float32, dev)
    _require(S0, "S0", (B, Hv, D, D), torch.float32, dev)
    if o is None or ST is None:
        raise ValueError("gdr_chunk_fwd_noalloc: o and ST are the caller's")
    _require(o, "o", (B, T, Hv, D), io_t, dev)
    _require(ST, "ST", (B, Hv, D, D), torch.float32, dev)
    desc = make_desc(B, T, Hqk, Hv, D, _io_dtype(q), _decay_of(g, (B, T), Hv, D), scale, chunk)
    _check(lib.gdr_chunk_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(b),
                                     _ptr(w), _ptr(S0), _ptr(o), _ptr(ST), _stream(stream)))
    return o, ST


def gdr_norm_la_workspace_bytes(desc: gdr_desc) -> int:
    n = ctypes.c_size_t()
    _check(lib.gdr_norm_la_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def gdr_norm_la_fwd(phq, phk, v, *, S0=None, z0=None, o=None, ST=None, zT=None, workspace=None, stream=None):
    """Normalised linear attention over the T tokens of phq [B,T,Hqk,D]
    (phi already applied to q and k). Returns (o, ST, zT); ST may be S0 and
    zT may be z0 for an in-place update."""
    torch = _torch()
    B, T, Hqk, D = phq.shape
    Hv = v.shape[2]
    dev, io_t = phq.device, phq.dtype
    for name, t, shape in (("phq", phq, (B, T, Hqk, D)), ("phk", phk, (B, T, Hqk, D)), ("v", v, (B, T, Hv, D))):
        _require(t, name, shape, io_t, dev)
    _require(S0, "S0", (B, Hv, D, D), torch.float32, dev)
    _require(z0, "z0", (B, Hv, D), torch.float32, dev)
    desc = make_desc(B, T, Hqk, Hv, D, _io_dtype(phq), GDR_DECAY_NONE)
    s = _torch_stream(stream, dev)
    with torch.cuda.stream(s):  # tensors made here belong to the stream the call runs on
        if o is None:
            o = torch.empty((B, T, Hv, D), dtype=io_t, device=dev)
        if ST is None:
            ST = torch.empty((B, Hv, D, D), dtype=torch.float32, device=dev)
        if zT is None:
            zT = torch.empty((B, Hv, D), dtype=torch.float32, device=dev)
        nbytes = gdr_norm_la_workspace_bytes(desc)
        if workspace is None and nbytes > 0:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _require(o, "o", (B, T, Hv, D), io_t, dev)
    _require(ST, "ST", (B, Hv, D, D), torch.float32, dev)
    _require(zT, "zT", (B, Hv, D), torch.float32, dev)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.gdr_norm_la_fwd(ctypes.byref(desc), _ptr(phq), _ptr(phk), _ptr(v), _ptr(S0), _ptr(z0), _ptr(o),
                               _ptr(ST), _ptr(zT), _ptr(workspace), wsz, _stream(s)))
    return o, ST, zT


def gdr_norm_la_decode_step(phq, phk, v, S, z, *, o=None, stream=None):
    """One normalised linear-attention step per sequence: phq, phk [B,Hqk,D],
    v [B,Hv,D]; S [B,Hv,D,D] and z [B,Hv,D] updated in place. Returns o."""
    torch = _torch()
    B, Hqk, D = phq.shape
    Hv = v.shape[1]
    dev, io_t = phq.device, phq.dtype
    for name, t, shape in (("phq", phq, (B, Hqk, D)), ("phk", phk, (B, Hqk, D)), ("v", v, (B, Hv, D))):
        _require(t, name, shape, io_t, dev)
    _require(S, "S", (B, Hv, D, D), torch.float32, dev)
    _require(z, "z", (B, Hv, D), torch.float32, dev)
    desc = make_desc(B, 1, Hqk, Hv, D, _io_dtype(phq), GDR_DECAY_NONE)
    s = _torch_stream(stream, dev)
    if o is None:
        with torch.cuda.stream(s):
            o = torch.empty((B, Hv, D), dtype=io_t, device=dev)
    _require(o, "o", (B, Hv, D), io_t, dev)
    _check(lib.gdr_norm_la_decode_step(ctypes.byref(desc), _ptr(phq), _ptr(phk), _ptr(v), _ptr(S), _ptr(z), _ptr(o),
                                       _stream(s)))
    return o


def gdr_decode_step(q, k, v, S, *, g=None, beta=None, b=None, w=None, scale=1.0, o=None, stream=None):
    """One decode step, updating S [B,Hv,D,D] in place. Returns o [B,Hv,D]."""
    torch = _torch()
    B, Hqk, D = q.shape
    Hv = v.shape[1]
    dev, io_t = q.device, q.dtype
    for name, t, shape in (("q", q, (B, Hqk, D)), ("k", k, (B, Hqk, D)), ("v", v, (B, Hv, D)),
                           ("b", b, (B, Hv, D)), ("w", w, (B, Hv, D))):
        _require(t, name, shape, io_t, dev)
    _require(beta, "beta", (B, Hv), torch.float32, dev)
    _require(g, "g", None, torch.float32, dev)
    _require(S, "S", (B, Hv, D, D), torch.float32, dev)
    desc = make_desc(B, 1, Hqk, Hv, D, _io_dtype(q), _decay_of(g, (B,), Hv, D), scale)
    s = _torch_stream(stream, dev)
    if o is None:
        with torch.cuda.stream(s):
            o = torch.empty((B, Hv, D), dtype=io_t, device=dev)
    _require(o, "o", (B, Hv, D), io_t, dev)
    _check(lib.gdr_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(b),
                               _ptr(w), _ptr(S), _ptr(o), _stream(s)))
    return o


def gdr_recurrent_fwd(q, k, v, *, g=None, beta=None, b=None, w=None, S0=None, scale=1.0, o=None, ST=None,
                      stream=None):
    """Fused recurrent forward over the T tokens of q [B,T,Hqk,D] from S0
    (None = zeros). Returns (o, ST); ST may be passed equal to S0 for an
    in-place state update. Same layouts and results as gdr_chunk_fwd."""
    torch = _torch()
    B, T, Hqk, D = q.shape
    Hv = v.shape[2]
    dev, io_t = q.device, q.dtype
    for name, t, shape in (("q", q, (B, T, Hqk, D)), ("k", k, (B, T, Hqk, D)), ("v", v, (B, T, Hv, D)),
                           ("b", b, (B, T, Hv, D)), ("w", w, (B, T, Hv, D))):
        _require(t, name, shape, io_t, dev)
    _require(beta, "beta", (B, T, Hv), torch.float32, dev)
    _require(g, "g", None, torch.float32, dev)
    _require(S0, "S0", (B, Hv, D, D), torch.float32, dev)
    desc = make_desc(B, T, Hqk, Hv, D, _io_dtype(q), _decay_of(g, (B, T), Hv, D), scale)
    s = _torch_stream(stream, dev)
    with torch.cuda.stream(s):
        if o is None:
            o = torch.empty((B, T, Hv, D), dtype=io_t, device=dev)
        if ST is None:
            ST = torch.empty((B, Hv, D, D), dtype=torch.float32, device=dev)
    _require(o, "o", (B, T, Hv, D), io_t, dev)
    _require(ST, "ST", (B, Hv, D, D), torch.float32, dev)
    _check(lib.gdr_recurrent_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(b),
                                 _ptr(w), _ptr(S0), _ptr(o), _ptr(ST), _stream(s)))
    return o, ST


def _stage_args(q, v, conv_w, conv_in, conv_out, decay_scale):
    """Shared checks of the input-stage arguments; returns (stage struct,
    conv_out tensor or None)."""
    torch = _torch()
    B, _, Hqk, D = q.shape
    Hv = v.shape[2]
    ch = (2 * Hqk + Hv) * D
    _require(conv_in, "conv_in", (B, 3, ch), q.dtype, q.device)
    _require(conv_w, "conv_w", (ch, 4), torch.float32, q.device)
    _require(decay_scale, "decay_scale", (Hv,), torch.float32, q.device)
    if conv_out is None:
        conv_out = torch.empty((B, 3, ch), dtype=q.dtype, device=q.device)
    elif conv_out is False:
        conv_out = None
    _require(conv_out, "conv_out", (B, 3, ch), q.dtype, q.device)
    return gdr_input_stage(_ptr(conv_w), _ptr(conv_in), _ptr(conv_out), _ptr(decay_scale)), conv_out


def gdr_chunk_fwd_in(q, k, v, conv_w, *, conv_in=None, conv_out=None, decay_scale=None, g=None, beta=None, b=None,
                     w=None, S0=None, scale=1.0, chunk=CHUNK, o=None, ST=None, workspace=None, stream=None):
    """gdr_chunk_fwd with the input stage fused into its load stage; the
    arguments of gdr_recurrent_fwd_in plus the workspace. Returns (o, ST,
    conv_out)."""
    torch = _torch()
    B, T, Hqk, D = q.shape
    Hv = v.shape[2]
    dev, io_t = q.device, q.dtype
    for name, t, shape in (("q", q, (B, T, Hqk, D)), ("k", k, (B, T, Hqk, D)), ("v", v, (B, T, Hv, D)),
                           ("b", b, (B, T, Hv, D)), ("w", w, (B, T, Hv, D))):
        _require(t, name, shape, io_t, dev)
    _require(beta, "beta", (B, T, Hv), torch.float32, dev)
    _require(g, "g", None, torch.float32, dev)
    _require(S0, "S0", (B, Hv, D, D), torch.float32, dev)
    desc = make_desc(B, T, Hqk, Hv, D, _io_dtype(q), _decay_of(g, (B, T), Hv, D), scale, chunk)
    s = _torch_stream(stream, dev)
    with torch.cuda.stream(s):
        stage, conv_out = _stage_args(q, v, conv_w, conv_in, conv_out, decay_scale)
        if o is None:
            o = torch.empty((B, T, Hv, D), dtype=io_t, device=dev)
        if ST is None:
            ST = torch.empty((B, Hv, D, D), dtype=torch.float32, device=dev)
        nbytes = gdr_chunk_fwd_in_workspace_bytes(desc)
        if workspace is None and nbytes > 0:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _require(o, "o", (B, T, Hv, D), io_t, dev)
    _require(ST, "ST", (B, Hv, D, D), torch.float32, dev)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.gdr_chunk_fwd_in(ctypes.byref(desc), ctypes.byref(stage), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                _ptr(beta), _ptr(b), _ptr(w), _ptr(S0), _ptr(o), _ptr(ST), _ptr(workspace), wsz,
                                _stream(s)))
    return o, ST, conv_out


def gdr_recurrent_fwd_in(q, k, v, conv_w, *, conv_in=None, conv_out=None, decay_scale=None, g=None, beta=None,
                         b=None, w=None, S0=None, scale=1.0, o=None, ST=None, stream=None):
    """gdr_recurrent_fwd with the input stage fused in: q [B,T,Hqk,D], k, v
    are raw projections; beta, b, w gate inputs before the sigmoid; g the
    decay input before -c softplus; conv_w [(2 Hqk + Hv) D, 4] float32 taps;
    conv_in [B, 3, (2 Hqk + Hv) D] (io dtype) or None for zeros; decay_scale
    [Hv] float32 or None. Returns (o, ST, conv_out); conv_out (the last 3 raw
    tokens) is allocated when None and not written when False."""
    torch = _torch()
    B, T, Hqk, D = q.shape
    Hv = v.shape[2]
    dev, io_t = q.device, q.dtype
    for name, t, shape in (("q", q, (B, T, Hqk, D)), ("k", k, (B, T, Hqk, D)), ("v", v, (B, T, Hv, D)),
                           ("b", b, (B, T, Hv, D)), ("w", w, (B, T, Hv, D))):
        _require(t, name, shape, io_t, dev)
    _require(beta, "beta", (B, T, Hv), torch.float32, dev)
    _require(g, "g", None, torch.float32, dev)
    _require(S0, "S0", (B, Hv, D, D), torch.float32, dev)
    desc = make_desc(B, T, Hqk, Hv, D, _io_dtype(q), _decay_of(g, (B, T), Hv, D), scale)
    s = _torch_stream(stream, dev)
    with torch.cuda.stream(s):
        if o is None:
            o = torch.empty((B, T, Hv, D), dtype=io_t, device=dev)
        if ST is None:
            ST = torch.empty((B, Hv, D, D), dtype=torch.float32, device=dev)
        stage, conv_out = _stage_args(q, v, conv_w, conv_in, conv_out, decay_scale)
    _require(o, "o", (B, T, Hv, D), io_t, dev)
    _require(ST, "ST", (B, Hv, D, D), torch.float32, dev)
    _check(lib.gdr_recurrent_fwd_in(ctypes.byref(desc), ctypes.byref(stage), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                    _ptr(beta), _ptr(b), _ptr(w), _ptr(S0), _ptr(o), _ptr(ST), _stream(s)))
    return o, ST, conv_out


def gdr_recurrent_bwd_workspace_bytes(desc: gdr_desc) -> int:
    n = ctypes.c_size_t()
    _check(lib.gdr_recurrent_bwd_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def gdr_chunk_bwd_workspace_bytes(desc: gdr_desc) -> int:
    n = ctypes.c_size_t()
    _check(lib.gdr_chunk_bwd_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def gdr_recurrent_bwd(q, k, v, do, *, g=None, beta=None, b=None, w=None, S0=None, dST=None, scale=1.0,
                      want_dS0=True, workspace=None, stream=None):
    """Gradients of the recurrence for dL/do = do [B,T,Hv,D] (io dtype) and
    dL/dS_T = dST ([B,Hv,D,D] float32, or None for zeros). Inputs as given to
    the forward call. Returns a dict of float32 tensors: dq, dk, dv, and dg,
    dbeta, db, dw, dS0 where they apply (dS0 only when want_dS0)."""
    return _bwd(False, q, k, v, do, g, beta, b, w, S0, dST, scale, want_dS0, workspace, stream)


def gdr_chunk_bwd(q, k, v, do, *, g=None, beta=None, b=None, w=None, S0=None, dST=None, scale=1.0,
                  want_dS0=True, workspace=None, stream=None):
    """gdr_recurrent_bwd's gradients in chunked form (parallel over chunks of
    64 tokens); same arguments and result."""
    return _bwd(True, q, k, v, do, g, beta, b, w, S0, dST, scale, want_dS0, workspace, stream)


def _bwd(chunked, q, k, v, do, g, beta, b, w, S0, dST, scale, want_dS0, workspace, stream):
    torch = _torch()
    B, T, Hqk, D = q.shape
    Hv = v.shape[2]
    dev, io_t = q.device, q.dtype
    for name, t, shape in (("q", q, (B, T, Hqk, D)), ("k", k, (B, T, Hqk, D)), ("v", v, (B, T, Hv, D)),
                           ("b", b, (B, T, Hv, D)), ("w", w, (B, T, Hv, D)), ("do", do, (B, T, Hv, D))):
        _require(t, name, shape, io_t, dev)
    _require(beta, "beta", (B, T, Hv), torch.float32, dev)
    _require(g, "g", None, torch.float32, dev)
    _require(S0, "S0", (B, Hv, D, D), torch.float32, dev)
    _require(dST, "dST", (B, Hv, D, D), torch.float32, dev)
    desc = make_desc(B, T, Hqk, Hv, D, _io_dtype(q), _decay_of(g, (B, T), Hv, D), scale)
    f32 = dict(dtype=torch.float32, device=dev)
    s = _torch_stream(stream, dev)
    with torch.cuda.stream(s):
        out = {"dq": torch.empty((B, T, Hqk, D), **f32), "dk": torch.empty((B, T, Hqk, D), **f32),
               "dv": torch.empty((B, T, Hv, D), **f32)}
        if g is not None:
            out["dg"] = torch.empty(g.shape, **f32)
        if beta is not None:
            out["dbeta"] = torch.empty((B, T, Hv), **f32)
        if b is not None:
            out["db"] = torch.empty((B, T, Hv, D), **f32)
            out["dw"] = torch.empty((B, T, Hv, D), **f32)
        if want_dS0:
            out["dS0"] = torch.empty((B, Hv, D, D), **f32)
        nbytes = (gdr_chunk_bwd_workspace_bytes if chunked else gdr_recurrent_bwd_workspace_bytes)(desc)
        if workspace is None and nbytes > 0:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = lib.gdr_chunk_bwd if chunked else lib.gdr_recurrent_bwd
    _check(fn(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(b), _ptr(w), _ptr(S0),
              _ptr(do), _ptr(dST), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out.get("dg")),
              _ptr(out.get("dbeta")), _ptr(out.get("db")), _ptr(out.get("dw")), _ptr(out.get("dS0")),
              _ptr(workspace), wsz, _stream(s)))
    return out
