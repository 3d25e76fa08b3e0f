"""libmssm: MI355X-native (gfx950) selective-scan forward.

The compute lives in hand-written HIP kernels behind a C ABI
(``include/mssm.h``, built into ``libmssm.so`` in this package directory).
This package only marshals torch tensors (device memory and the current HIP
stream) into that ABI; it computes nothing itself.

The library is loaded on first use; if it is missing or fails to load, the
call raises -- there is no CPU fallback.
"""
from .api import (  # noqa: F401
    MssmError,
    selective_scan_bwd,
    selective_scan_conv_fwd,
    selective_scan_fwd,
    selective_scan_fwd_noalloc,
    selective_state_update,
    ssd_scalar_fwd,
    version,
)

__all__ = ["MssmError", "selective_scan_bwd", "selective_scan_conv_fwd", "selective_scan_fwd",
           "selective_scan_fwd_noalloc", "selective_state_update",
           "ssd_scalar_fwd", "version"]
