"""Pins of the oracle's selective-scan backward (CPU only).

The backward is checked against directional central differences of the
forward oracle (itself pinned to closed forms elsewhere): for a random loss
l = sum(dy * y) + sum(dh_last * h_last) and a random direction v in one
input at a time, sum(grad * v) must equal (l(x + e v) - l(x - e v)) / 2e.
Planted mistakes in a copy of the backward must each fail that pin.
"""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

from oracle import oracle
from selective_state_space_05_amd import inputs

ORACLE_C = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "oracle.c")

GRAD_OF = {"u": "du", "delta": "ddelta", "delta_bias": "ddelta_bias", "A": "dA", "B": "dB",
           "C": "dC", "D": "dD", "z": "dz", "h0": "dh0"}


def _problem(seed, gate=True, batch=2, L=11, dim=3, N=4):
    p = inputs.ScanProblem("b", batch, L, dim, N, "f32", "per_channel", gate, True, seed)
    x = {k: (None if v is None else v.astype(np.float64)) for k, v in inputs.scan_inputs(p).items()
         if k not in ("conv_w", "conv_b")}
    rng = np.random.default_rng(seed + 100)
    x["h0"] = rng.standard_normal((batch, dim, N))
    dy = rng.standard_normal((batch, dim, L))
    dhl = rng.standard_normal((batch, dim, N))
    return x, dy, dhl


def _loss(x, dy, dhl, lib=None):
    y, h = oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"],
                                 x["delta_bias"], h0=x["h0"], lib=lib)
    return float(np.sum(dy * y) + np.sum(dhl * h))


def _fd_failures(lib=None, seed=3, gate=True, eps=1e-5, tol=1e-6):
    x, dy, dhl = _problem(seed, gate)
    g = oracle.selective_scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"],
                                  z=x["z"], delta_bias=x["delta_bias"], h0=x["h0"],
                                  dh_last=dhl, lib=lib)
    rng = np.random.default_rng(seed + 7)
    failed = []
    for name, gname in GRAD_OF.items():
        if x[name] is None:
            continue
        v = rng.standard_normal(x[name].shape)
        xp, xm = dict(x), dict(x)
        xp[name] = x[name] + eps * v
        xm[name] = x[name] - eps * v
        fd = (_loss(xp, dy, dhl) - _loss(xm, dy, dhl)) / (2 * eps)
        an = float(np.sum(g[gname] * v))
        if not abs(fd - an) <= tol * max(1.0, abs(an)):
            failed.append((name, fd, an))
    return failed


@pytest.mark.parametrize("gate", [True, False])
@pytest.mark.parametrize("seed", [3, 4])
def test_backward_matches_central_differences(gate, seed):
    assert _fd_failures(seed=seed, gate=gate) == []


def test_backward_without_optional_inputs():
    """No bias, skip, gate, initial state or final-state gradient: the
    required gradients are unchanged in form and still match differences."""
    p = inputs.ScanProblem("b", 1, 9, 2, 3, "f32", None, False, False, 5)
    x = {k: (None if v is None else v.astype(np.float64)) for k, v in inputs.scan_inputs(p).items()}
    dy = np.random.default_rng(1).standard_normal(x["u"].shape)
    g = oracle.selective_scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy)
    assert g["dD"] is None and g["dz"] is None and g["ddelta_bias"] is None and g["dh0"] is None
    rng = np.random.default_rng(2)
    for name in ("u", "delta", "A", "B", "C"):
        v = rng.standard_normal(x[name].shape)
        lo = {k: x[k] for k in ("u", "delta", "A", "B", "C")}
        hi = dict(lo)
        lo[name] = x[name] - 1e-5 * v
        hi[name] = x[name] + 1e-5 * v
        f = lambda a: float(np.sum(dy * oracle.selective_scan(a["u"], a["delta"], a["A"], a["B"],   # noqa: E731
                                                               a["C"])[0]))
        fd = (f(hi) - f(lo)) / 2e-5
        an = float(np.sum(g[GRAD_OF[name]] * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), name


def test_skip_gradient_closed_form():
    """y is affine in D with slope u * silu(z): dD = sum dy u silu(z)."""
    x, dy, dhl = _problem(9)
    g = oracle.selective_scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"],
                                  z=x["z"], delta_bias=x["delta_bias"], h0=x["h0"], dh_last=dhl)
    silu = x["z"] / (1.0 + np.exp(-x["z"]))
    ref = np.sum(dy * x["u"] * silu, axis=(0, 2))
    assert np.max(np.abs(g["dD"] - ref)) <= 1e-12 * np.max(np.abs(ref))


BWD_MUTANTS = {
    "identity": [],
    "dA_missing_dl": [("gA[d * N + n] += dh[n] * hprev * a * dl;", "gA[d * N + n] += dh[n] * hprev * a;")],
    "carry_not_decayed": [("                dh[n] *= a;\n", "")],
    "state_index_shifted": [("double hprev = hist[t * N + n];", "double hprev = hist[(t + 1) * N + n];")],
    "gate_derivative_sigmoid_only": [("dyt * s * sz * (1.0 + zt * (1.0 - sz))", "dyt * s * sz")],
    "ddelta_without_sigmoid": [("ddelta[r * L + t] = ddl * sig;", "ddelta[r * L + t] = ddl;")],
    "dB_missing_u": [("gB[b * N * L + n * L + t] += dh[n] * dl * ur[t];",
                      "gB[b * N * L + n * L + t] += dh[n] * dl;")],
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(tmp_path, name):
    src = open(ORACLE_C).read()
    for old, new in BWD_MUTANTS[name]:
        assert old in src, "mutation anchor not found: %r" % old
        src = src.replace(old, new)
    c = os.path.join(str(tmp_path), name + ".c")
    so = os.path.join(str(tmp_path), name + ".so")
    with open(c, "w") as f:
        f.write(src)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", "-std=c99",
                    c, "-o", so, "-lm"], check=True)
    lib = oracle.load_variant(so)
    failed = _fd_failures(lib=lib)
    if name == "identity":
        assert failed == []
    else:
        assert failed, "mutant %s passed the difference pin" % name
