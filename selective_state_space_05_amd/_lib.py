"""ctypes declaration of the libmssm C ABI (``include/mssm.h``).

Argument marshalling only.  The library is looked up next to this file;
if it is absent or fails to load, :func:`lib` raises -- there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmssm.so")

MSSM_OK = 0
MSSM_ERR_INVALID_ARG = 1
MSSM_ERR_UNSUPPORTED = 2
MSSM_ERR_HIP = 3
MSSM_ERR_ALLOC = 4

MSSM_F32 = 0
MSSM_BF16 = 1

VARIANT_AUTO = 0
VARIANT_ROWSERIAL = 1
VARIANT_CHUNKED = 2
VARIANT_LOOKBACK = 3
VARIANT_SSD_RECURRENT = 4
VARIANT_SSD_CHUNKED = 5
VARIANT_PAIRSCAN = 6
VARIANT_PAIRSCAN2 = 7

MAX_DSTATE = 64
DEVICE_LOOKBACK_TIMEOUT = 0x1   # mssm_device_status bit
NOALLOC_SCRATCH_BYTES = 8 << 20  # scratch array of the no-alloc entry point
CONV_WIDTH = 4
SSD_MAX_DSTATE = 256
SSD_MAX_HEADDIM = 256

# Every symbol the header declares.
EXPORTED = (
    "mssm_selective_scan_fwd",
    "mssm_ssd_scalar_fwd",
    "mssm_selective_scan_fwd_h0",
    "mssm_selective_scan_fwd_conv",
    "mssm_selective_scan_bwd",
    "mssm_ssd_scalar_fwd_h0",
    "mssm_ssd_scalar_fwd_gated",
    "mssm_selective_state_update",
    "mssm_force_variant",
    "mssm_last_variant",
    "mssm_status_string",
    "mssm_last_error",
    "mssm_version",
    "mssm_source_hash",
    "mssm_device_status",
    "mssm_selective_scan_fwd_h0_noalloc",
)
# Every symbol include/mssm_probes.h declares (measurement probes).
EXPORTED_PROBES = (
    "mssm_probe_copy",
    "mssm_probe_valu",
)
PROBE_FMA, PROBE_EXP2, PROBE_LOG2, PROBE_RCP = 0, 1, 2, 3
PROBE_VALU_THREADS = 2048 * 256
PROBE_VALU_OPS_PER_ITER = 128


class ScanDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("dim", ctypes.c_int64), ("dstate", ctypes.c_int64)]


class SSDDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk", ctypes.c_int64)]


class StepDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("dim", ctypes.c_int64),
                ("dstate", ctypes.c_int64)]


class DTypes(ctypes.Structure):
    _fields_ = [("io", ctypes.c_int32), ("param", ctypes.c_int32)]


_lock = threading.Lock()
_lib = None


def _declare(L):
    vp = ctypes.c_void_p
    fp = ctypes.c_void_p          # float* passed as raw device addresses
    L.mssm_selective_scan_fwd.argtypes = [vp, vp, fp, fp, vp, vp, fp, vp, vp,
                                          fp, ScanDims, DTypes, vp]
    L.mssm_selective_scan_fwd.restype = ctypes.c_int
    L.mssm_ssd_scalar_fwd.argtypes = [vp, vp, fp, fp, vp, vp, fp, vp, fp,
                                      SSDDims, DTypes, vp]
    L.mssm_ssd_scalar_fwd.restype = ctypes.c_int
    L.mssm_selective_scan_fwd_h0.argtypes = [vp, vp, fp, fp, vp, vp, fp, vp, fp,
                                             vp, fp, ScanDims, DTypes, vp]
    L.mssm_selective_scan_fwd_h0.restype = ctypes.c_int
    L.mssm_selective_scan_fwd_h0_noalloc.argtypes = [vp, vp, fp, fp, vp, vp, fp, vp, fp,
                                                     vp, fp, ScanDims, DTypes, vp]
    L.mssm_selective_scan_fwd_h0_noalloc.restype = ctypes.c_int
    L.mssm_selective_scan_fwd_conv.argtypes = [vp, fp, fp, vp, fp, fp, vp, vp, fp, vp, fp,
                                               vp, fp, ScanDims, DTypes, vp]
    L.mssm_selective_scan_fwd_conv.restype = ctypes.c_int
    L.mssm_selective_scan_bwd.argtypes = [vp, vp, fp, fp, vp, vp, fp, vp, fp, vp, fp,
                                          vp, vp, fp, fp, fp, fp, fp, vp, fp,
                                          ScanDims, DTypes, vp]
    L.mssm_selective_scan_bwd.restype = ctypes.c_int
    L.mssm_ssd_scalar_fwd_h0.argtypes = [vp, vp, fp, fp, vp, vp, fp, fp, vp, fp,
                                         SSDDims, DTypes, vp]
    L.mssm_ssd_scalar_fwd_h0.restype = ctypes.c_int
    L.mssm_ssd_scalar_fwd_gated.argtypes = [vp, vp, fp, fp, vp, vp, fp, vp, fp, vp, fp,
                                            SSDDims, DTypes, vp]
    L.mssm_ssd_scalar_fwd_gated.restype = ctypes.c_int
    L.mssm_selective_state_update.argtypes = [fp, vp, vp, fp, fp, vp, vp, fp, vp, vp,
                                              StepDims, DTypes, vp]
    L.mssm_selective_state_update.restype = ctypes.c_int
    L.mssm_force_variant.argtypes = [ctypes.c_int]
    L.mssm_force_variant.restype = ctypes.c_int
    L.mssm_last_variant.argtypes = []
    L.mssm_last_variant.restype = ctypes.c_int
    L.mssm_status_string.argtypes = [ctypes.c_int]
    L.mssm_status_string.restype = ctypes.c_char_p
    L.mssm_last_error.argtypes = []
    L.mssm_last_error.restype = ctypes.c_char_p
    L.mssm_version.argtypes = []
    L.mssm_version.restype = ctypes.c_int
    L.mssm_probe_copy.argtypes = [vp, vp, ctypes.c_int64, vp]
    L.mssm_probe_copy.restype = ctypes.c_int
    L.mssm_probe_valu.argtypes = [ctypes.c_int, ctypes.c_int32, fp, vp]
    L.mssm_probe_valu.restype = ctypes.c_int
    L.mssm_source_hash.argtypes = []
    L.mssm_source_hash.restype = ctypes.c_char_p
    L.mssm_device_status.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int]
    L.mssm_device_status.restype = ctypes.c_int
    return L


class StaleLibraryError(OSError):
    """The library was built from sources other than those beside it."""


def check_source_hash(L):
    """Refuse a library built from other sources than the ones in this
    package (a stale binary would silently run old kernels)."""
    from . import build
    if not os.path.isdir(build.CSRC):
        return
    want = build.source_hash()
    got = L.mssm_source_hash().decode()
    if got != want:
        raise StaleLibraryError(
            "libmssm.so was built from other sources (library %s, sources %s): rebuild it "
            "(python -c 'import __graft_entry__ as g; g.build()')" % (got, want))


def load(path: str = LIB_PATH):
    """Load and declare a libmssm build (raises OSError if it cannot)."""
    if not os.path.exists(path):
        raise OSError(
            "libmssm.so not found at %s: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()')" % path)
    L = _declare(ctypes.CDLL(path))
    check_source_hash(L)
    return L


def lib():
    global _lib
    with _lock:
        if _lib is None:
            _lib = load()
    return _lib
