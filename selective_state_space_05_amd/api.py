"""torch-tensor front end of libmssm.

Each function checks tensor metadata, allocates the outputs with torch
(device memory), and passes raw device pointers plus the current HIP stream
to the C ABI.  No arithmetic of the method happens here.
"""
from __future__ import annotations

import contextlib

import torch

from . import _lib


class MssmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_status_name(status), message))
        self.status = status


def _status_name(s: int) -> str:
    try:
        return _lib.lib().mssm_status_string(s).decode()
    except OSError:
        return "status %d" % s


def _check(status: int):
    if status != _lib.MSSM_OK:
        msg = _lib.lib().mssm_last_error().decode()
        raise MssmError(status, msg)


def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return _lib.MSSM_F32
    if t.dtype == torch.bfloat16:
        return _lib.MSSM_BF16
    raise TypeError("activations must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, dtype=None, device=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if device is not None and t.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, t.device))


def _need_shape(t, name, shape):
    """Caller-supplied output buffers must have exactly the output's shape:
    the C ABI sees only their addresses, so a smaller buffer would be written
    past its end on the device."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _stream_handle(device):
    return torch.cuda.current_stream(device).cuda_stream


def version() -> int:
    return int(_lib.lib().mssm_version())


@contextlib.contextmanager
def forced_variant(variant: int):
    """Run the enclosed calls (on this thread) with a fixed kernel variant."""
    L = _lib.lib()
    prev = L.mssm_force_variant(int(variant))
    try:
        yield
    finally:
        L.mssm_force_variant(prev)


def last_variant() -> int:
    return int(_lib.lib().mssm_last_variant())


def device_status(clear: bool = False) -> int:
    """Status bits the library's kernels set on the current device
    (``_lib.DEVICE_LOOKBACK_TIMEOUT``); waits for the device first."""
    import ctypes
    bits = ctypes.c_uint32(0)
    _check(_lib.lib().mssm_device_status(ctypes.byref(bits), 1 if clear else 0))
    return int(bits.value)


def selective_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                       return_last_state=True, out=None, h_out=None, h0=None):
    """Selective-scan forward on the GPU.

    u, delta, z: (batch, dim, L) float32 or bfloat16 (all the same dtype);
    B, C: (batch, N, L) same dtype; A: (dim, N) float32; D, delta_bias:
    (dim,) float32; h0: (batch, dim, N) float32 initial state (None: zero;
    it may be passed as ``h_out`` too, to advance a state in place).
    Returns ``(y, h_last)`` with y like u and h_last (batch, dim, N) float32
    (None if ``return_last_state`` is False).
    """
    L = _lib.lib()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    io = u.dtype
    for name, t in (("u", u), ("delta", delta), ("B", B), ("C", C), ("z", z)):
        _need(t, name, io, dev)
    for name, t in (("A", A), ("D", D), ("delta_bias", delta_bias), ("h0", h0)):
        _need(t, name, torch.float32, dev)
    batch, dim, seqlen = u.shape
    N = A.shape[1]
    if h0 is not None and tuple(h0.shape) != (batch, dim, N):
        raise ValueError("h0 must be (batch, dim, N)")
    if delta.shape != u.shape or (z is not None and z.shape != u.shape):
        raise ValueError("u, delta, z must share one (batch, dim, L) shape")
    if tuple(A.shape) != (dim, N):
        raise ValueError("A must be (dim, N)")
    if tuple(B.shape) != (batch, N, seqlen) or tuple(C.shape) != (batch, N, seqlen):
        raise ValueError("B and C must be (batch, N, L)")
    for name, t in (("D", D), ("delta_bias", delta_bias)):
        if t is not None and tuple(t.shape) != (dim,):
            raise ValueError("%s must be (dim,)" % name)
    _need_shape(out, "out", u.shape)
    _need_shape(h_out, "h_out", (batch, dim, N))
    y = out if out is not None else torch.empty_like(u)
    _need(y, "out", io, dev)
    h_last = None
    if return_last_state:
        h_last = h_out if h_out is not None else torch.empty(
            (batch, dim, N), dtype=torch.float32, device=dev)
        _need(h_last, "h_out", torch.float32, dev)
    dims = _lib.ScanDims(batch, seqlen, dim, N)
    dt = _lib.DTypes(_io_dtype(u), _lib.MSSM_F32)
    with torch.cuda.device(dev):
        if h0 is None:
            st = L.mssm_selective_scan_fwd(
                _ptr(u), _ptr(delta), _ptr(delta_bias), _ptr(A), _ptr(B), _ptr(C),
                _ptr(D), _ptr(z), _ptr(y), _ptr(h_last), dims, dt,
                _stream_handle(dev))
        else:
            st = L.mssm_selective_scan_fwd_h0(
                _ptr(u), _ptr(delta), _ptr(delta_bias), _ptr(A), _ptr(B), _ptr(C),
                _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(h_last), dims, dt,
                _stream_handle(dev))
    _check(st)
    return y, h_last


def selective_scan_fwd_noalloc(u, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None,
                               *, out, h_out):
    """``selective_scan_fwd`` through the entry point that allocates nothing
    on the device (mssm_selective_scan_fwd_h0_noalloc): the caller passes
    the outputs ``out`` (like u) and ``h_out`` ((batch, dim, N) float32,
    or None), and scratch comes from the library's fixed per-device array.
    Calls that overlap on one device race on that array."""
    L = _lib.lib()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    io = u.dtype
    for name, t in (("u", u), ("delta", delta), ("B", B), ("C", C), ("z", z)):
        _need(t, name, io, dev)
    for name, t in (("A", A), ("D", D), ("delta_bias", delta_bias), ("h0", h0)):
        _need(t, name, torch.float32, dev)
    if out is None:
        raise ValueError("out is required")
    batch, dim, seqlen = u.shape
    N = A.shape[1]
    if delta.shape != u.shape or (z is not None and z.shape != u.shape):
        raise ValueError("u, delta, z must share one (batch, dim, L) shape")
    if tuple(A.shape) != (dim, N):
        raise ValueError("A must be (dim, N)")
    if tuple(B.shape) != (batch, N, seqlen) or tuple(C.shape) != (batch, N, seqlen):
        raise ValueError("B and C must be (batch, N, L)")
    for name, t in (("D", D), ("delta_bias", delta_bias)):
        if t is not None and tuple(t.shape) != (dim,):
            raise ValueError("%s must be (dim,)" % name)
    for name, t in (("h0", h0), ("h_out", h_out)):
        _need_shape(t, name, (batch, dim, N))
    _need_shape(out, "out", u.shape)
    _need(out, "out", io, dev)
    _need(h_out, "h_out", torch.float32, dev)
    dims = _lib.ScanDims(batch, seqlen, dim, N)
    dtp = _lib.DTypes(_io_dtype(u), _lib.MSSM_F32)
    with torch.cuda.device(dev):
        st = L.mssm_selective_scan_fwd_h0_noalloc(
            _ptr(u), _ptr(delta), _ptr(delta_bias), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
            _ptr(z), _ptr(h0), _ptr(out), _ptr(h_out), dims, dtp, _stream_handle(dev))
    _check(st)
    return out, h_out


def selective_scan_conv_fwd(x, conv_w, delta, A, B, C, D=None, z=None, delta_bias=None,
                            conv_b=None, h0=None, return_last_state=True, out=None, h_out=None):
    """Selective-scan forward fed by its convolution prologue on the GPU:
    the scan of u = silu(conv_b + causal width-4 depthwise conv(x)), with u
    formed on chip.

    x: (batch, dim, L) like the scan's u; conv_w: (dim, 4) float32; conv_b:
    (dim,) float32.  Other arguments and the result as for
    ``selective_scan_fwd``.
    """
    L = _lib.lib()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    _need(conv_w, "conv_w", torch.float32, dev)
    _need(conv_b, "conv_b", torch.float32, dev)
    batch, dim, seqlen = x.shape
    if tuple(conv_w.shape) != (dim, _lib.CONV_WIDTH):
        raise ValueError("conv_w must be (dim, %d)" % _lib.CONV_WIDTH)
    if conv_b is not None and tuple(conv_b.shape) != (dim,):
        raise ValueError("conv_b must be (dim,)")
    io = x.dtype
    for name, t in (("x", x), ("delta", delta), ("B", B), ("C", C), ("z", z)):
        _need(t, name, io, dev)
    for name, t in (("A", A), ("D", D), ("delta_bias", delta_bias), ("h0", h0)):
        _need(t, name, torch.float32, dev)
    N = A.shape[1]
    if delta.shape != x.shape or (z is not None and z.shape != x.shape):
        raise ValueError("x, delta, z must share one (batch, dim, L) shape")
    if tuple(A.shape) != (dim, N):
        raise ValueError("A must be (dim, N)")
    if tuple(B.shape) != (batch, N, seqlen) or tuple(C.shape) != (batch, N, seqlen):
        raise ValueError("B and C must be (batch, N, L)")
    if h0 is not None and tuple(h0.shape) != (batch, dim, N):
        raise ValueError("h0 must be (batch, dim, N)")
    for name, t in (("D", D), ("delta_bias", delta_bias)):
        if t is not None and tuple(t.shape) != (dim,):
            raise ValueError("%s must be (dim,)" % name)
    _need_shape(out, "out", x.shape)
    _need_shape(h_out, "h_out", (batch, dim, N))
    y = out if out is not None else torch.empty_like(x)
    _need(y, "out", io, dev)
    h_last = None
    if return_last_state:
        h_last = h_out if h_out is not None else torch.empty(
            (batch, dim, N), dtype=torch.float32, device=dev)
        _need(h_last, "h_out", torch.float32, dev)
    dims = _lib.ScanDims(batch, seqlen, dim, N)
    dtp = _lib.DTypes(_io_dtype(x), _lib.MSSM_F32)
    with torch.cuda.device(dev):
        st = L.mssm_selective_scan_fwd_conv(
            _ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(delta), _ptr(delta_bias), _ptr(A),
            _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(h_last), dims, dtp,
            _stream_handle(dev))
    _check(st)
    return y, h_last


def selective_scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, h0=None,
                       dh_last=None):
    """Gradients of the selective scan on the GPU for output gradients ``dy``
    (like u) and ``dh_last`` (batch, dim, N) float32 (None: zero).

    Returns a dict of float32 tensors: du, ddelta (batch, dim, L); dA
    (dim, N); dB, dC (batch, N, L); dD, ddelta_bias (dim,); dz (batch, dim,
    L, when z is given); dh0 (batch, dim, N).
    """
    L = _lib.lib()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    io = u.dtype
    for name, t in (("u", u), ("delta", delta), ("B", B), ("C", C), ("z", z), ("dy", dy)):
        _need(t, name, io, dev)
    for name, t in (("A", A), ("D", D), ("delta_bias", delta_bias), ("h0", h0),
                    ("dh_last", dh_last)):
        _need(t, name, torch.float32, dev)
    batch, dim, seqlen = u.shape
    N = A.shape[1]
    if delta.shape != u.shape or dy.shape != u.shape or (z is not None and z.shape != u.shape):
        raise ValueError("u, delta, z, dy must share one (batch, dim, L) shape")
    if tuple(A.shape) != (dim, N):
        raise ValueError("A must be (dim, N)")
    if tuple(B.shape) != (batch, N, seqlen) or tuple(C.shape) != (batch, N, seqlen):
        raise ValueError("B and C must be (batch, N, L)")
    for name, t in (("h0", h0), ("dh_last", dh_last)):
        if t is not None and tuple(t.shape) != (batch, dim, N):
            raise ValueError("%s must be (batch, dim, N)" % name)
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"du": torch.empty(u.shape, **f32), "ddelta": torch.empty(u.shape, **f32),
         "dA": torch.empty((dim, N), **f32), "dB": torch.empty((batch, N, seqlen), **f32),
         "dC": torch.empty((batch, N, seqlen), **f32), "dD": torch.empty((dim,), **f32),
         "ddelta_bias": torch.empty((dim,), **f32),
         "dz": None if z is None else torch.empty(u.shape, **f32),
         "dh0": torch.empty((batch, dim, N), **f32)}
    dims = _lib.ScanDims(batch, seqlen, dim, N)
    dtp = _lib.DTypes(_io_dtype(u), _lib.MSSM_F32)
    with torch.cuda.device(dev):
        st = L.mssm_selective_scan_bwd(
            _ptr(u), _ptr(delta), _ptr(delta_bias), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(h0), _ptr(dy), _ptr(dh_last), _ptr(g["du"]), _ptr(g["ddelta"]),
            _ptr(g["ddelta_bias"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]),
            _ptr(g["dz"]), _ptr(g["dh0"]), dims, dtp, _stream_handle(dev))
    _check(st)
    return g


def ssd_scalar_fwd(x, dt, A, B, C, D=None, dt_bias=None, chunk=0,
                   return_last_state=True, out=None, h_out=None, h0=None, z=None):
    """Mamba-2 scalar-decay forward on the GPU.

    x, z: (batch, L, H, P); dt: (batch, L, H); B, C: (batch, L, G, N), all
    in one activation dtype; A, D, dt_bias: (H,) float32; h0: (batch, H, P,
    N) float32 initial state (None: zero; may also be ``h_out``); z gates
    the output with silu(z) (None: no gate).  Returns ``(y, h_last)``: y
    like x, h_last (batch, H, P, N) float32.
    """
    L = _lib.lib()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    io = x.dtype
    for name, t in (("x", x), ("dt", dt), ("B", B), ("C", C), ("z", z)):
        _need(t, name, io, dev)
    for name, t in (("A", A), ("D", D), ("dt_bias", dt_bias), ("h0", h0)):
        _need(t, name, torch.float32, dev)
    batch, seqlen, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if h0 is not None and tuple(h0.shape) != (batch, H, P, N):
        raise ValueError("h0 must be (batch, H, P, N)")
    if z is not None and z.shape != x.shape:
        raise ValueError("z must be shaped like x")
    if tuple(dt.shape) != (batch, seqlen, H):
        raise ValueError("dt must be (batch, L, H)")
    if tuple(B.shape) != (batch, seqlen, G, N) or tuple(C.shape) != tuple(B.shape):
        raise ValueError("B and C must be (batch, L, G, N)")
    for name, t in (("A", A), ("D", D), ("dt_bias", dt_bias)):
        if t is not None and tuple(t.shape) != (H,):
            raise ValueError("%s must be (H,)" % name)
    _need_shape(out, "out", x.shape)
    _need_shape(h_out, "h_out", (batch, H, P, N))
    y = out if out is not None else torch.empty_like(x)
    _need(y, "out", io, dev)
    h_last = None
    if return_last_state:
        h_last = h_out if h_out is not None else torch.empty(
            (batch, H, P, N), dtype=torch.float32, device=dev)
        _need(h_last, "h_out", torch.float32, dev)
    dims = _lib.SSDDims(batch, seqlen, H, P, N, G, int(chunk))
    dtp = _lib.DTypes(_io_dtype(x), _lib.MSSM_F32)
    with torch.cuda.device(dev):
        if z is not None:
            st = L.mssm_ssd_scalar_fwd_gated(
                _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B), _ptr(C),
                _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(h_last), dims, dtp,
                _stream_handle(dev))
        elif h0 is None:
            st = L.mssm_ssd_scalar_fwd(
                _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B), _ptr(C),
                _ptr(D), _ptr(y), _ptr(h_last), dims, dtp, _stream_handle(dev))
        else:
            st = L.mssm_ssd_scalar_fwd_h0(
                _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B), _ptr(C),
                _ptr(D), _ptr(h0), _ptr(y), _ptr(h_last), dims, dtp,
                _stream_handle(dev))
    _check(st)
    return y, h_last


def selective_state_update(state, x, dt, A, B, C, D=None, z=None, dt_bias=None,
                           out=None):
    """One decode step on the GPU, advancing ``state`` in place.

    state: (batch, dim, N) float32; x, dt, z: (batch, dim) float32 or
    bfloat16 (one dtype); B, C: (batch, N) same dtype; A: (dim, N) float32;
    D, dt_bias: (dim,) float32.  Returns y (batch, dim) like x.
    """
    L = _lib.lib()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    io = x.dtype
    for name, t in (("x", x), ("dt", dt), ("B", B), ("C", C), ("z", z)):
        _need(t, name, io, dev)
    for name, t in (("state", state), ("A", A), ("D", D), ("dt_bias", dt_bias)):
        _need(t, name, torch.float32, dev)
    if x.dim() != 2:
        raise ValueError("x must be (batch, dim)")
    batch, dim = x.shape
    N = A.shape[1]
    if tuple(state.shape) != (batch, dim, N):
        raise ValueError("state must be (batch, dim, N)")
    if tuple(dt.shape) != (batch, dim) or (z is not None and tuple(z.shape) != (batch, dim)):
        raise ValueError("dt and z must be (batch, dim)")
    if tuple(A.shape) != (dim, N):
        raise ValueError("A must be (dim, N)")
    if tuple(B.shape) != (batch, N) or tuple(C.shape) != (batch, N):
        raise ValueError("B and C must be (batch, N)")
    for name, t in (("D", D), ("dt_bias", dt_bias)):
        if t is not None and tuple(t.shape) != (dim,):
            raise ValueError("%s must be (dim,)" % name)
    _need_shape(out, "out", x.shape)
    y = out if out is not None else torch.empty_like(x)
    _need(y, "out", io, dev)
    dims = _lib.StepDims(batch, dim, N)
    dtp = _lib.DTypes(_io_dtype(x), _lib.MSSM_F32)
    with torch.cuda.device(dev):
        st = L.mssm_selective_state_update(
            _ptr(state), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B), _ptr(C),
            _ptr(D), _ptr(z), _ptr(y), dims, dtp, _stream_handle(dev))
    _check(st)
    return y


def probe_copy(src, dst):
    """Launch the streaming copy probe (mssm_probe_copy) from ``src`` to
    ``dst`` (contiguous device tensors of the same byte size) on the current
    stream."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must hold the same number of bytes")
    _need(src, "src")
    _need(dst, "dst")
    with torch.cuda.device(src.device):
        _check(_lib.lib().mssm_probe_copy(_ptr(src), _ptr(dst), nbytes,
                                          _stream_handle(src.device)))


def probe_valu(op: int, iters: int, out):
    """Launch the ALU issue-rate probe (mssm_probe_valu) for operation ``op``
    (``_lib.PROBE_*``); ``out`` is a float32 device tensor of at least
    ``_lib.PROBE_VALU_THREADS`` elements.  Returns the lane-operations the
    launch performs."""
    _need(out, "out", torch.float32)
    if out.numel() < _lib.PROBE_VALU_THREADS:
        raise ValueError("out needs %d elements" % _lib.PROBE_VALU_THREADS)
    with torch.cuda.device(out.device):
        _check(_lib.lib().mssm_probe_valu(int(op), int(iters), _ptr(out),
                                          _stream_handle(out.device)))
    return _lib.PROBE_VALU_THREADS * int(iters) * _lib.PROBE_VALU_OPS_PER_ITER
