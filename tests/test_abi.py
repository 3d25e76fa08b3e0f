"""The C ABI without a GPU: the library loads, exports what include/mssm.h
declares, and rejects every invalid call before touching the HIP runtime.

Pointers here are fake non-null addresses: validation never dereferences
them, and no call in this file reaches a kernel launch.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

import pytest

from selective_state_space_05_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mssm.h")


@pytest.fixture(scope="module")
def L():
    """The library, built first when it is missing or was built from other
    sources (no GPU is needed to build or to run these tests)."""
    try:
        return _lib.lib()
    except OSError:
        from selective_state_space_05_amd import build
        build.build()
        _lib._lib = None
        return _lib.lib()


PROBES_HEADER = os.path.join(ROOT, "include", "mssm_probes.h")


def header_functions(path=None):
    """Functions declared by one header, or by every header under include/."""
    paths = [path] if path else [os.path.join(ROOT, "include", f)
                                 for f in sorted(os.listdir(os.path.join(ROOT, "include")))
                                 if f.endswith(".h")]
    names = set()
    for p in paths:
        names |= set(re.findall(r"MSSM_API\s+[\w\s\*]+?\b(mssm_\w+)\s*\(", open(p).read()))
    return sorted(names)


def test_header_declares_expected_functions():
    assert header_functions(HEADER) == sorted(_lib.EXPORTED)
    assert header_functions(PROBES_HEADER) == sorted(_lib.EXPORTED_PROBES)


def test_library_exports_every_declared_symbol(L):
    for name in header_functions():
        assert hasattr(L, name), name


def test_only_the_c_abi_is_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert {s for s in syms if s.startswith("mssm")} == set(_lib.EXPORTED) | set(_lib.EXPORTED_PROBES)
    assert not [s for s in syms if s.startswith("_ZN4mssm")]


def test_header_constants_match_binding():
    src = open(HEADER).read()
    assert int(re.search(r"#define MSSM_MAX_DSTATE (\d+)", src).group(1)) == _lib.MAX_DSTATE
    assert int(re.search(r"#define MSSM_SSD_MAX_DSTATE (\d+)", src).group(1)) == _lib.SSD_MAX_DSTATE
    assert int(re.search(r"#define MSSM_SSD_MAX_HEADDIM (\d+)", src).group(1)) == _lib.SSD_MAX_HEADDIM
    assert int(re.search(r"#define MSSM_CONV_WIDTH (\d+)", src).group(1)) == _lib.CONV_WIDTH


def test_version_and_status_strings(L):
    assert L.mssm_version() >= 100
    for s, name in [(0, b"MSSM_OK"), (1, b"MSSM_ERR_INVALID_ARG"), (2, b"MSSM_ERR_UNSUPPORTED"),
                    (3, b"MSSM_ERR_HIP"), (4, b"MSSM_ERR_ALLOC")]:
        assert L.mssm_status_string(s) == name
    assert L.mssm_status_string(99) == b"MSSM_ERR_UNKNOWN"


# fake device addresses, far apart so ranges never overlap by accident
BASE = 0x7F0000000000
def fake(i):
    return BASE + i * (1 << 36)


def scan_call(L, batch=2, seqlen=64, dim=8, dstate=4, io=0, param=0, **ptrs):
    p = dict(u=fake(1), delta=fake(2), delta_bias=fake(3), A=fake(4), B=fake(5),
             C=fake(6), D=fake(7), z=fake(8), y=fake(9), h_last=fake(10))
    p.update(ptrs)
    return L.mssm_selective_scan_fwd(
        p["u"], p["delta"], p["delta_bias"], p["A"], p["B"], p["C"], p["D"],
        p["z"], p["y"], p["h_last"], _lib.ScanDims(batch, seqlen, dim, dstate),
        _lib.DTypes(io, param), None)


def ssd_call(L, batch=2, seqlen=64, H=4, P=8, N=16, G=1, chunk=0, io=0, param=0, **ptrs):
    p = dict(x=fake(1), dt=fake(2), dt_bias=fake(3), A=fake(4), B=fake(5), C=fake(6),
             D=fake(7), y=fake(9), h_last=fake(10))
    p.update(ptrs)
    return L.mssm_ssd_scalar_fwd(
        p["x"], p["dt"], p["dt_bias"], p["A"], p["B"], p["C"], p["D"], p["y"],
        p["h_last"], _lib.SSDDims(batch, seqlen, H, P, N, G, chunk),
        _lib.DTypes(io, param), None)


def scan_h0_call(L, batch=2, seqlen=64, dim=8, dstate=4, io=0, param=0, **ptrs):
    p = dict(u=fake(1), delta=fake(2), delta_bias=fake(3), A=fake(4), B=fake(5),
             C=fake(6), D=fake(7), z=fake(8), h0=fake(11), y=fake(9), h_last=fake(10))
    p.update(ptrs)
    return L.mssm_selective_scan_fwd_h0(
        p["u"], p["delta"], p["delta_bias"], p["A"], p["B"], p["C"], p["D"],
        p["z"], p["h0"], p["y"], p["h_last"], _lib.ScanDims(batch, seqlen, dim, dstate),
        _lib.DTypes(io, param), None)


def ssd_h0_call(L, batch=2, seqlen=64, H=4, P=8, N=16, G=1, chunk=0, io=0, param=0, **ptrs):
    p = dict(x=fake(1), dt=fake(2), dt_bias=fake(3), A=fake(4), B=fake(5), C=fake(6),
             D=fake(7), h0=fake(11), y=fake(9), h_last=fake(10))
    p.update(ptrs)
    return L.mssm_ssd_scalar_fwd_h0(
        p["x"], p["dt"], p["dt_bias"], p["A"], p["B"], p["C"], p["D"], p["h0"], p["y"],
        p["h_last"], _lib.SSDDims(batch, seqlen, H, P, N, G, chunk),
        _lib.DTypes(io, param), None)


def scan_conv_call(L, batch=2, seqlen=64, dim=8, dstate=4, io=0, param=0, **ptrs):
    p = dict(x=fake(1), conv_w=fake(12), conv_b=fake(13), delta=fake(2), delta_bias=fake(3),
             A=fake(4), B=fake(5), C=fake(6), D=fake(7), z=fake(8), h0=fake(11), y=fake(9),
             h_last=fake(10))
    p.update(ptrs)
    return L.mssm_selective_scan_fwd_conv(
        p["x"], p["conv_w"], p["conv_b"], p["delta"], p["delta_bias"], p["A"], p["B"], p["C"],
        p["D"], p["z"], p["h0"], p["y"], p["h_last"], _lib.ScanDims(batch, seqlen, dim, dstate),
        _lib.DTypes(io, param), None)


def bwd_call(L, batch=2, seqlen=64, dim=8, dstate=4, io=0, param=0, **ptrs):
    names = ["u", "delta", "delta_bias", "A", "B", "C", "D", "z", "h0", "dy", "dh_last", "du",
             "ddelta", "ddelta_bias", "dA", "dB", "dC", "dD", "dz", "dh0"]
    p = {n: fake(30 + i) for i, n in enumerate(names)}
    p.update(ptrs)
    return L.mssm_selective_scan_bwd(*[p[n] for n in names], _lib.ScanDims(batch, seqlen, dim, dstate),
                                     _lib.DTypes(io, param), None)


def ssd_gated_call(L, batch=2, seqlen=64, H=4, P=8, N=16, G=1, chunk=0, io=0, param=0, **ptrs):
    p = dict(x=fake(1), dt=fake(2), dt_bias=fake(3), A=fake(4), B=fake(5), C=fake(6),
             D=fake(7), z=fake(8), h0=fake(11), y=fake(9), h_last=fake(10))
    p.update(ptrs)
    return L.mssm_ssd_scalar_fwd_gated(
        p["x"], p["dt"], p["dt_bias"], p["A"], p["B"], p["C"], p["D"], p["z"], p["h0"],
        p["y"], p["h_last"], _lib.SSDDims(batch, seqlen, H, P, N, G, chunk),
        _lib.DTypes(io, param), None)


def step_call(L, batch=2, dim=8, dstate=4, io=0, param=0, **ptrs):
    p = dict(state=fake(10), x=fake(1), dt=fake(2), dt_bias=fake(3), A=fake(4), B=fake(5),
             C=fake(6), D=fake(7), z=fake(8), y=fake(9))
    p.update(ptrs)
    return L.mssm_selective_state_update(
        p["state"], p["x"], p["dt"], p["dt_bias"], p["A"], p["B"], p["C"], p["D"], p["z"],
        p["y"], _lib.StepDims(batch, dim, dstate), _lib.DTypes(io, param), None)


@pytest.mark.parametrize("name", ["u", "delta", "A", "B", "C", "y"])
def test_scan_null_required_pointer(L, name):
    assert scan_call(L, **{name: None}) == _lib.MSSM_ERR_INVALID_ARG
    assert name.encode() in L.mssm_last_error()


@pytest.mark.parametrize("dims", [dict(batch=-1), dict(seqlen=-5), dict(dim=-2),
                                  dict(dstate=0), dict(dstate=-3)])
def test_scan_bad_sizes(L, dims):
    assert scan_call(L, **dims) == _lib.MSSM_ERR_INVALID_ARG
    assert L.mssm_last_error()


def test_scan_size_overflow(L):
    assert scan_call(L, batch=1 << 40, seqlen=1 << 30, dim=1 << 10) == _lib.MSSM_ERR_INVALID_ARG
    assert b"overflow" in L.mssm_last_error()


def test_scan_dstate_limit(L):
    assert scan_call(L, dstate=_lib.MAX_DSTATE + 1) == _lib.MSSM_ERR_UNSUPPORTED


@pytest.mark.parametrize("io,param,status", [(2, 0, 1), (-1, 0, 1), (0, 7, 1), (0, 1, 2)])
def test_scan_dtypes(L, io, param, status):
    assert scan_call(L, io=io, param=param) == status


@pytest.mark.parametrize("out,inp", [("y", "u"), ("y", "delta"), ("y", "z"), ("y", "B"),
                                     ("h_last", "A"), ("h_last", "C"), ("y", "D")])
def test_scan_output_aliasing_input(L, out, inp):
    assert scan_call(L, **{out: fake(20), inp: fake(20) + 8}) == _lib.MSSM_ERR_INVALID_ARG
    assert b"overlaps" in L.mssm_last_error()


def test_scan_y_overlapping_h_last(L):
    assert scan_call(L, y=fake(20), h_last=fake(20) + 64) == _lib.MSSM_ERR_INVALID_ARG


def test_scan_adjacent_buffers_do_not_alias(L):
    # u occupies [fake(20), fake(20) + 2*8*64*4); y starts right after it.
    nbytes = 2 * 8 * 64 * 4
    with_variant = L.mssm_force_variant(_lib.VARIANT_SSD_RECURRENT)
    try:
        st = scan_call(L, u=fake(20), y=fake(20) + nbytes)
    finally:
        L.mssm_force_variant(with_variant)
    # passes validation; stops at the variant check, before any launch
    assert st == _lib.MSSM_ERR_UNSUPPORTED
    assert b"variant" in L.mssm_last_error()


def test_scan_empty_problem_is_noop(L):
    assert scan_call(L, batch=0) == _lib.MSSM_OK
    assert scan_call(L, dim=0, u=None, y=None) == _lib.MSSM_OK
    # L == 0 without h_last: nothing to write, no launch
    assert scan_call(L, seqlen=0, u=None, delta=None, B=None, C=None, y=None,
                     h_last=None) == _lib.MSSM_OK


def test_scan_h0_overlapping_an_output(L):
    # h0 is an input: no output may overlap it ...
    assert scan_h0_call(L, h0=fake(20), y=fake(20) + 4) == _lib.MSSM_ERR_INVALID_ARG
    assert b"h0" in L.mssm_last_error()
    # ... except h_last being the very same buffer (state advanced in place)
    assert scan_h0_call(L, h0=fake(20), h_last=fake(20) + 16) == _lib.MSSM_ERR_INVALID_ARG
    prev = L.mssm_force_variant(_lib.VARIANT_SSD_RECURRENT)
    try:
        st = scan_h0_call(L, h0=fake(20), h_last=fake(20))
    finally:
        L.mssm_force_variant(prev)
    assert st == _lib.MSSM_ERR_UNSUPPORTED      # validation passed; stopped at the variant
    assert b"variant" in L.mssm_last_error()


def test_scan_h0_validation_matches_scan(L):
    for kw in (dict(u=None), dict(dstate=0), dict(batch=-1), dict(io=3)):
        assert scan_h0_call(L, **kw) == scan_call(L, **kw) == _lib.MSSM_ERR_INVALID_ARG
    assert scan_h0_call(L, dstate=_lib.MAX_DSTATE + 1) == _lib.MSSM_ERR_UNSUPPORTED
    assert scan_h0_call(L, batch=0) == _lib.MSSM_OK
    # L == 0 with the state kept in place: nothing to copy, no launch
    assert scan_h0_call(L, seqlen=0, u=None, delta=None, B=None, C=None, y=None,
                        h0=fake(20), h_last=fake(20)) == _lib.MSSM_OK


def test_ssd_h0_overlapping_an_output(L):
    assert ssd_h0_call(L, h0=fake(20), y=fake(20) + 2) == _lib.MSSM_ERR_INVALID_ARG
    assert ssd_h0_call(L, h0=fake(20), h_last=fake(20) + 4) == _lib.MSSM_ERR_INVALID_ARG
    prev = L.mssm_force_variant(_lib.VARIANT_CHUNKED)
    try:
        st = ssd_h0_call(L, h0=fake(20), h_last=fake(20))
    finally:
        L.mssm_force_variant(prev)
    assert st == _lib.MSSM_ERR_UNSUPPORTED
    assert b"variant" in L.mssm_last_error()
    assert ssd_h0_call(L, seqlen=0, h0=fake(20), h_last=fake(20)) == _lib.MSSM_OK


def test_scan_conv_validation(L):
    assert scan_conv_call(L, conv_w=None) == _lib.MSSM_ERR_INVALID_ARG
    assert b"conv_w" in L.mssm_last_error()
    assert scan_conv_call(L, x=None) == _lib.MSSM_ERR_INVALID_ARG
    assert scan_conv_call(L, dstate=_lib.MAX_DSTATE + 1) == _lib.MSSM_ERR_UNSUPPORTED
    # the taps are inputs: outputs may not overlap them
    assert scan_conv_call(L, conv_w=fake(20), y=fake(20) + 8) == _lib.MSSM_ERR_INVALID_ARG
    assert scan_conv_call(L, conv_b=fake(20), h_last=fake(20)) == _lib.MSSM_ERR_INVALID_ARG
    prev = L.mssm_force_variant(_lib.VARIANT_SSD_RECURRENT)
    try:
        st = scan_conv_call(L, conv_b=None, h0=None, z=None)
    finally:
        L.mssm_force_variant(prev)
    assert st == _lib.MSSM_ERR_UNSUPPORTED       # validation passed; stopped at the variant
    assert b"variant" in L.mssm_last_error()


@pytest.mark.parametrize("name", ["u", "delta", "A", "B", "C", "dy", "du", "ddelta"])
def test_bwd_null_required_pointer(L, name):
    assert bwd_call(L, **{name: None}) == _lib.MSSM_ERR_INVALID_ARG
    assert name.encode() in L.mssm_last_error()


def test_bwd_validation(L):
    assert bwd_call(L, z=None) == _lib.MSSM_ERR_INVALID_ARG        # dz without z
    assert b"dz" in L.mssm_last_error()
    assert bwd_call(L, dstate=0) == _lib.MSSM_ERR_INVALID_ARG
    assert bwd_call(L, dstate=_lib.MAX_DSTATE + 1) == _lib.MSSM_ERR_UNSUPPORTED
    assert bwd_call(L, io=7) == _lib.MSSM_ERR_INVALID_ARG
    assert bwd_call(L, batch=1 << 40, seqlen=1 << 30) == _lib.MSSM_ERR_INVALID_ARG
    # gradients are outputs: none may overlap an input or another output
    assert bwd_call(L, du=fake(50), dy=fake(50) + 8) == _lib.MSSM_ERR_INVALID_ARG
    assert bwd_call(L, dB=fake(50), dC=fake(50) + 16) == _lib.MSSM_ERR_INVALID_ARG
    assert bwd_call(L, dA=fake(50), A=fake(50)) == _lib.MSSM_ERR_INVALID_ARG
    assert b"overlaps" in L.mssm_last_error()


def test_ssd_gated_validation(L):
    assert ssd_gated_call(L, x=None) == _lib.MSSM_ERR_INVALID_ARG
    assert ssd_gated_call(L, H=6, G=4) == _lib.MSSM_ERR_INVALID_ARG
    assert ssd_gated_call(L, N=257) == _lib.MSSM_ERR_UNSUPPORTED
    # the gate is an input: no output may overlap it
    assert ssd_gated_call(L, z=fake(20), y=fake(20) + 2) == _lib.MSSM_ERR_INVALID_ARG
    assert b"z" in L.mssm_last_error()
    assert ssd_gated_call(L, z=fake(20), h_last=fake(20) + 4) == _lib.MSSM_ERR_INVALID_ARG
    assert ssd_gated_call(L, batch=0) == _lib.MSSM_OK
    prev = L.mssm_force_variant(_lib.VARIANT_CHUNKED)
    try:
        st = ssd_gated_call(L, z=None, h0=None)
    finally:
        L.mssm_force_variant(prev)
    assert st == _lib.MSSM_ERR_UNSUPPORTED       # optional z and h0 both absent: validation passes
    assert b"variant" in L.mssm_last_error()


@pytest.mark.parametrize("name", ["state", "x", "dt", "A", "B", "C", "y"])
def test_step_null_required_pointer(L, name):
    assert step_call(L, **{name: None}) == _lib.MSSM_ERR_INVALID_ARG
    assert name.encode() in L.mssm_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), 1), (dict(dim=-1), 1), (dict(dstate=0), 1), (dict(io=4), 1),
    (dict(param=1), 2), (dict(dstate=_lib.MAX_DSTATE + 1), 2),
    (dict(batch=1 << 40, dim=1 << 30), 1)])
def test_step_validation(L, kw, status):
    assert step_call(L, **kw) == status
    assert L.mssm_last_error()


@pytest.mark.parametrize("out,inp", [("y", "x"), ("y", "z"), ("state", "A"), ("state", "B"),
                                     ("state", "dt"), ("y", "D")])
def test_step_output_aliasing_input(L, out, inp):
    assert step_call(L, **{out: fake(20), inp: fake(20) + 2}) == _lib.MSSM_ERR_INVALID_ARG
    assert b"overlaps" in L.mssm_last_error()


def test_step_y_overlapping_state(L):
    assert step_call(L, y=fake(20), state=fake(20) + 8) == _lib.MSSM_ERR_INVALID_ARG


def test_step_empty_problem_is_noop(L):
    assert step_call(L, batch=0) == _lib.MSSM_OK
    assert step_call(L, dim=0, state=None, x=None, y=None) == _lib.MSSM_OK


@pytest.mark.parametrize("name", ["x", "dt", "A", "B", "C", "y"])
def test_ssd_null_required_pointer(L, name):
    assert ssd_call(L, **{name: None}) == _lib.MSSM_ERR_INVALID_ARG
    assert name.encode() in L.mssm_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(H=6, G=4), 1), (dict(G=0), 1), (dict(chunk=-1), 1), (dict(P=0), 1),
    (dict(N=0), 1), (dict(batch=-1), 1), (dict(P=257), 2), (dict(N=257), 2),
    (dict(io=5), 1), (dict(param=1), 2)])
def test_ssd_validation(L, kw, status):
    assert ssd_call(L, **kw) == status
    assert L.mssm_last_error()


def test_ssd_chunked_refuses_grids_past_its_limit(L):
    """The matrix-core SSD form launches one workgroup of 256 work-items per
    (batch, chunk pair, head, 64-column slice); a grid of 2^24 or more such
    workgroups would pass 2^32 work-items, so the forced variant refuses the
    shape before any launch (here 2^15 x 1 x 1024 x 1 workgroups)."""
    prev = L.mssm_force_variant(_lib.VARIANT_SSD_CHUNKED)
    try:
        st = ssd_call(L, batch=1 << 15, seqlen=64, H=1024, P=8, N=16, io=1)
    finally:
        L.mssm_force_variant(prev)
    assert st == _lib.MSSM_ERR_UNSUPPORTED
    assert b"variant" in L.mssm_last_error()


def test_ssd_output_aliasing(L):
    assert ssd_call(L, y=fake(20), x=fake(20) + 2) == _lib.MSSM_ERR_INVALID_ARG
    assert ssd_call(L, h_last=fake(20), B=fake(20) + 4) == _lib.MSSM_ERR_INVALID_ARG


def test_ssd_empty_problem_is_noop(L):
    assert ssd_call(L, batch=0) == _lib.MSSM_OK
    assert ssd_call(L, seqlen=0, h_last=None) == _lib.MSSM_OK


def test_force_variant_returns_previous_and_is_thread_local(L):
    prev = L.mssm_force_variant(_lib.VARIANT_ROWSERIAL)
    try:
        seen = []
        th = threading.Thread(target=lambda: seen.append(L.mssm_force_variant(0)))
        th.start()
        th.join()
        assert seen == [_lib.VARIANT_AUTO]
        assert L.mssm_force_variant(_lib.VARIANT_ROWSERIAL) == _lib.VARIANT_ROWSERIAL
    finally:
        L.mssm_force_variant(prev)


def test_last_error_is_thread_local(L):
    assert scan_call(L, u=None) == _lib.MSSM_ERR_INVALID_ARG
    mine = L.mssm_last_error()
    other = []

    def worker():
        other.append(L.mssm_last_error())
        ssd_call(L, x=None)
        other.append(L.mssm_last_error())

    th = threading.Thread(target=worker)
    th.start()
    th.join()
    assert other[0] == b"" and b"x is null" in other[1]
    assert L.mssm_last_error() == mine


def test_binding_refuses_cpu_tensors():
    import torch
    import selective_state_space_05_amd as mssm
    u = torch.zeros(1, 2, 4)
    with pytest.raises(ValueError):
        mssm.selective_scan_fwd(u, u, torch.zeros(2, 4), torch.zeros(1, 4, 4),
                                torch.zeros(1, 4, 4))


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(OSError):
        _lib.load(str(tmp_path / "libmssm.so"))


def test_library_built_from_these_sources(L):
    """The loaded binary carries the hash of the sources beside it."""
    from selective_state_space_05_amd import build
    assert L.mssm_source_hash().decode() == build.source_hash()


def test_binding_refuses_a_stale_library(monkeypatch):
    """A library whose embedded hash differs from the sources' is refused."""
    from selective_state_space_05_amd import build
    monkeypatch.setattr(build, "source_hash", lambda: "0" * 16)
    with pytest.raises(_lib.StaleLibraryError):
        _lib.load()


def test_device_status_rejects_null(L):
    assert L.mssm_device_status(None, 0) == _lib.MSSM_ERR_INVALID_ARG
    assert b"bits is null" in L.mssm_last_error()


def test_device_status_bit_matches_header():
    src = open(HEADER).read()
    assert int(re.search(r"#define MSSM_DEVICE_LOOKBACK_TIMEOUT (0x[0-9a-f]+)u", src).group(1),
               16) == _lib.DEVICE_LOOKBACK_TIMEOUT


def test_noalloc_rejects_scratch_beyond_its_array(L):
    """Forced to the look-back variant, a problem of 5000 channel groups
    would need about 10 MB of scratch: refused before anything is queued."""
    prev = L.mssm_force_variant(_lib.VARIANT_LOOKBACK)
    try:
        p = [fake(i) for i in range(1, 12)]
        st = L.mssm_selective_scan_fwd_h0_noalloc(
            p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], None, p[8], p[9],
            _lib.ScanDims(1, 4096, 16 * 5000, 16), _lib.DTypes(1, 0), None)
    finally:
        L.mssm_force_variant(prev)
    assert st == _lib.MSSM_ERR_UNSUPPORTED
    assert b"no-alloc" in L.mssm_last_error()


def test_noalloc_validation_matches_scan(L):
    """The no-alloc entry point validates exactly like the allocating one."""
    p = [fake(i) for i in range(1, 12)]
    dims = _lib.ScanDims(2, 64, 8, 4)
    dt = _lib.DTypes(0, 0)
    for args in ([None] + p[1:8] + [None, p[8], p[9]],
                 p[:8] + [None, None, p[9]],
                 p[:8] + [None, p[0], p[9]]):
        a = L.mssm_selective_scan_fwd_h0(*args, dims, dt, None)
        b = L.mssm_selective_scan_fwd_h0_noalloc(*args, dims, dt, None)
        assert a == b != 0


def test_noalloc_scratch_size_matches_header():
    src = open(HEADER).read()
    assert re.search(r"#define MSSM_NOALLOC_SCRATCH_BYTES \(8u << 20\)", src)
    assert _lib.NOALLOC_SCRATCH_BYTES == 8 << 20


def test_probe_constants_match_binding():
    src = open(PROBES_HEADER).read()
    for name, val in (("FMA", _lib.PROBE_FMA), ("EXP2", _lib.PROBE_EXP2),
                      ("LOG2", _lib.PROBE_LOG2), ("RCP", _lib.PROBE_RCP)):
        assert int(re.search(r"#define MSSM_PROBE_%s (\d+)" % name, src).group(1)) == val
    assert re.search(r"#define MSSM_PROBE_VALU_THREADS \(2048 \* 256\)", src)
    assert _lib.PROBE_VALU_THREADS == 2048 * 256
    assert int(re.search(r"#define MSSM_PROBE_VALU_OPS_PER_ITER (\d+)", src).group(1)) == \
        _lib.PROBE_VALU_OPS_PER_ITER


def test_probe_validation(L):
    assert L.mssm_probe_copy(None, fake(2), 1024, None) == _lib.MSSM_ERR_INVALID_ARG
    assert L.mssm_probe_copy(fake(1), fake(2), 1000, None) == _lib.MSSM_ERR_INVALID_ARG
    assert L.mssm_probe_copy(fake(1), fake(1) + 512, 1024, None) == _lib.MSSM_ERR_INVALID_ARG
    assert b"overlap" in L.mssm_last_error()
    assert L.mssm_probe_copy(fake(1) + 4, fake(2), 1024, None) == _lib.MSSM_ERR_INVALID_ARG
    assert L.mssm_probe_valu(7, 10, fake(1), None) == _lib.MSSM_ERR_INVALID_ARG
    assert L.mssm_probe_valu(0, 0, fake(1), None) == _lib.MSSM_ERR_INVALID_ARG
    assert L.mssm_probe_valu(0, 10, None, None) == _lib.MSSM_ERR_INVALID_ARG
