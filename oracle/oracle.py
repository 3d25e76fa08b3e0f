"""Python face of the float64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product path never
imports this module.  It shares nothing with the HIP library; the two meet
only in the seeded input generator, which holds none of the method's
arithmetic.

Every input is converted exactly to float64 from the very values the GPU
receives (float32, or bfloat16 held as float32), so the oracle and the GPU
see identical operands.

Definitions (see ``oracle.c`` for the step-by-step loops):
  * ``selective_scan`` — per-step ZOH decay exp(delta*A), deltaB_u =
    delta*B*u, softplus(delta+bias), output C.h + D*u, optional silu(z) gate;
    "Mamba状态空间模型的硬件感知推理优化" (ybb.press) sections 1 and 3.1,
    www.mhpq.cn/news/984979 essay section 2.2.
  * ``ssd`` — Mamba-2 scalar per-step decay shared by all state elements of a
    head; same ybb.press page, section 4.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` with gcc (float64, no FMA contraction, OpenMP)."""
    if (not force and os.path.exists(_LIB_PATH)
            and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC)):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-shared", "-fPIC", "-std=c99", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(path: str):
    """Load a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    i64 = ctypes.c_int64
    lib.oracle_selective_scan_f64.argtypes = [
        i64, i64, i64, i64, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
        _dp, _dp, _dp, ctypes.c_int]
    lib.oracle_selective_scan_f64.restype = None
    lib.oracle_ssd_f64.argtypes = [
        i64, i64, i64, i64, i64, i64, _dp, _dp, _dp, _dp, _dp, _dp,
        _dp, _dp, _dp, _dp, _dp, ctypes.c_int]
    lib.oracle_ssd_f64.restype = None
    lib.oracle_selective_scan_bwd_f64.argtypes = [i64, i64, i64, i64] + [_dp] * 20
    lib.oracle_selective_scan_bwd_f64.restype = None
    lib.oracle_conv1d_silu_f64.argtypes = [i64, i64, i64, i64, _dp, _dp, _dp, _dp]
    lib.oracle_conv1d_silu_f64.restype = None
    lib.oracle_softplus_f64.argtypes = [ctypes.c_double]
    lib.oracle_softplus_f64.restype = ctypes.c_double
    lib.oracle_silu_f64.argtypes = [ctypes.c_double]
    lib.oracle_silu_f64.restype = ctypes.c_double
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = _bind(_LIB_PATH)
    return _lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def softplus(x: float) -> float:
    return _load().oracle_softplus_f64(float(x))


def silu(z: float) -> float:
    return _load().oracle_silu_f64(float(z))


def load_variant(path: str):
    """Bind another build of ``oracle.c`` (tests build edited copies of the
    source to show that the pins catch planted mistakes)."""
    return _bind(path)


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                   h0=None, nthreads: int = 0, lib=None):
    """Float64 selective scan.  Returns ``(y, h_last)``.

    u, delta, z: (batch, Dch, L); B, C: (batch, N, L); A: (Dch, N);
    D, delta_bias: (Dch,); h0: (batch, Dch, N).  ``nthreads`` <= 0 uses every
    OpenMP thread; results do not depend on it.  ``lib`` selects a library
    bound by ``load_variant`` (default: the oracle).
    """
    u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
    D, z, delta_bias, h0 = map(_f64, (D, z, delta_bias, h0))
    batch, Dch, L = u.shape
    N = A.shape[1]
    assert delta.shape == u.shape and A.shape == (Dch, N)
    assert B.shape == (batch, N, L) and C.shape == (batch, N, L)
    assert z is None or z.shape == u.shape
    assert D is None or D.shape == (Dch,)
    assert delta_bias is None or delta_bias.shape == (Dch,)
    assert h0 is None or h0.shape == (batch, Dch, N)
    if N > 1024:
        raise ValueError("oracle supports N <= 1024")
    y = np.empty((batch, Dch, L), np.float64)
    h_last = np.empty((batch, Dch, N), np.float64)
    (lib or _load()).oracle_selective_scan_f64(
        batch, L, Dch, N, _ptr(u), _ptr(delta), _ptr(delta_bias), _ptr(A),
        _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(h_last),
        int(nthreads))
    return y, h_last


def selective_scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, h0=None,
                       dh_last=None, lib=None):
    """Float64 gradients of the selective scan for output gradients ``dy``
    (like u) and ``dh_last`` (batch, Dch, N; None -> 0).

    Returns a dict with du, ddelta, dA, dB, dC, and dD, dz, ddelta_bias,
    dh0 for the optional inputs that were given (None otherwise).
    """
    u, delta, A, B, C, dy = map(_f64, (u, delta, A, B, C, dy))
    D, z, delta_bias, h0, dh_last = map(_f64, (D, z, delta_bias, h0, dh_last))
    batch, Dch, L = u.shape
    N = A.shape[1]
    assert delta.shape == u.shape and dy.shape == u.shape and A.shape == (Dch, N)
    assert B.shape == (batch, N, L) and C.shape == (batch, N, L)
    assert z is None or z.shape == u.shape
    assert h0 is None or h0.shape == (batch, Dch, N)
    assert dh_last is None or dh_last.shape == (batch, Dch, N)
    out = {"du": np.empty_like(u), "ddelta": np.empty_like(u), "dA": np.empty_like(A),
           "dB": np.empty_like(B), "dC": np.empty_like(C),
           "dD": None if D is None else np.empty(Dch),
           "dz": None if z is None else np.empty_like(u),
           "ddelta_bias": None if delta_bias is None else np.empty(Dch),
           "dh0": None if h0 is None else np.empty((batch, Dch, N))}
    (lib or _load()).oracle_selective_scan_bwd_f64(
        batch, L, Dch, N, _ptr(u), _ptr(delta), _ptr(delta_bias), _ptr(A), _ptr(B), _ptr(C),
        _ptr(D), _ptr(z), _ptr(h0), _ptr(dy), _ptr(dh_last), _ptr(out["du"]),
        _ptr(out["ddelta"]), _ptr(out["ddelta_bias"]), _ptr(out["dA"]), _ptr(out["dB"]),
        _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dz"]), _ptr(out["dh0"]))
    return out


def conv1d_silu(x, conv_w, conv_b=None, lib=None):
    """Float64 causal depthwise convolution + SiLU: u = silu(conv_b + sum_k
    conv_w[:, k] * x[..., t - (K-1) + k]), zero before the first step.

    x: (batch, Dch, L); conv_w: (Dch, K); conv_b: (Dch,).  Returns u like x.
    """
    x, conv_w = _f64(x), _f64(conv_w)
    conv_b = _f64(conv_b)
    batch, Dch, L = x.shape
    K = conv_w.shape[1]
    assert conv_w.shape == (Dch, K)
    assert conv_b is None or conv_b.shape == (Dch,)
    u = np.empty_like(x)
    (lib or _load()).oracle_conv1d_silu_f64(batch, Dch, L, K, _ptr(x), _ptr(conv_w),
                                            _ptr(conv_b), _ptr(u))
    return u


def selective_scan_conv(x, conv_w, conv_b, delta, A, B, C, D=None, z=None, delta_bias=None,
                        h0=None, nthreads: int = 0, lib=None):
    """The selective scan fed by the convolution prologue: the scan of
    ``u = conv1d_silu(x, conv_w, conv_b)``, skip term D * u.  Returns
    ``(y, h_last)``."""
    u = conv1d_silu(x, conv_w, conv_b, lib=lib)
    return selective_scan(u, delta, A, B, C, D, z, delta_bias, h0=h0, nthreads=nthreads, lib=lib)


def selective_scan_rows(rows, u, delta, A, B, C, D=None, z=None,
                        delta_bias=None, nthreads: int = 0):
    """Oracle on a subset of independent (b, d) rows of a large problem.

    Each row of the selective scan depends only on its own inputs, so a
    sampled row is computed exactly as in the full problem.  Returns
    ``(y_rows (R, L), h_rows (R, N))`` in the order of ``rows``.
    """
    rows = [(int(b), int(d)) for b, d in rows]
    ys, hs = [], []
    for b, d in rows:
        y, h = selective_scan(
            u[b:b + 1, d:d + 1], delta[b:b + 1, d:d + 1], A[d:d + 1],
            B[b:b + 1], C[b:b + 1],
            None if D is None else D[d:d + 1],
            None if z is None else z[b:b + 1, d:d + 1],
            None if delta_bias is None else delta_bias[d:d + 1],
            nthreads=nthreads)
        ys.append(y[0, 0])
        hs.append(h[0, 0])
    return np.stack(ys), np.stack(hs)


def ssd(x, dt, A, B, C, D=None, dt_bias=None, h0=None, nthreads: int = 0,
        lib=None, z=None):
    """Float64 Mamba-2 scalar-decay scan.  Returns ``(y, h_last)``.

    x, z: (batch, L, H, P); dt: (batch, L, H); B, C: (batch, L, G, N);
    A, D, dt_bias: (H,); h0: (batch, H, P, N).  z (optional) gates the
    output with silu(z).
    """
    x, dt, A, B, C = map(_f64, (x, dt, A, B, C))
    D, dt_bias, h0, z = map(_f64, (D, dt_bias, h0, z))
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (batch, L, H) and A.shape == (H,)
    assert B.shape == (batch, L, G, N) and C.shape == B.shape
    assert H % G == 0
    assert D is None or D.shape == (H,)
    assert dt_bias is None or dt_bias.shape == (H,)
    assert h0 is None or h0.shape == (batch, H, P, N)
    assert z is None or z.shape == x.shape
    if P * N > 65536:
        raise ValueError("oracle supports P*N <= 65536")
    y = np.empty((batch, L, H, P), np.float64)
    h_last = np.empty((batch, H, P, N), np.float64)
    (lib or _load()).oracle_ssd_f64(
        batch, L, H, P, N, G, _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A),
        _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(h_last),
        int(nthreads))
    return y, h_last


def ssd_rows(rows, x, dt, A, B, C, D=None, dt_bias=None, nthreads: int = 0, z=None,
             h0=None):
    """Oracle on sampled independent (b, h, p) rows of a large SSD problem.

    With a scalar decay per (b, t, h), every headdim index p evolves its own
    N-vector of state, independent of the other p (h0, when given, supplies
    each row's own starting N-vector).  Returns
    ``(y_rows (R, L), h_rows (R, N))``.
    """
    ys, hs = [], []
    for b, h, p in rows:
        b, h, p = int(b), int(h), int(p)
        G = B.shape[2]
        g = h // (x.shape[2] // G)
        y, hl = ssd(
            x[b:b + 1, :, h:h + 1, p:p + 1], dt[b:b + 1, :, h:h + 1],
            A[h:h + 1], B[b:b + 1, :, g:g + 1], C[b:b + 1, :, g:g + 1],
            None if D is None else D[h:h + 1],
            None if dt_bias is None else dt_bias[h:h + 1],
            h0=None if h0 is None else h0[b:b + 1, h:h + 1, p:p + 1],
            nthreads=nthreads,
            z=None if z is None else z[b:b + 1, :, h:h + 1, p:p + 1])
        ys.append(y[0, :, 0, 0])
        hs.append(hl[0, 0, 0])
    return np.stack(ys), np.stack(hs)
