"""Planted mistakes in the oracle must fail a pin.

Each case copies ``oracle/oracle.c``, applies one plausible mistake (a
dropped term, a wrong sign, a shifted or transposed index, a missing
nonlinearity), builds it with gcc into a temporary directory and runs the
same pins the oracle passes.  Every mutant must fail at least one of them;
the unmodified copy must pass all.  CPU only; the real oracle is untouched.
"""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import pins
from oracle import oracle as oracle_py
from selective_state_space_05_amd import inputs

ORACLE_C = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "oracle.c")

SCAN_MUTANTS = {
    "identity": [],
    "drop_skip_term": [("double yv = acc + skip * ut;", "double yv = acc;")],
    "flip_sign_of_A": [("exp(dl * Ad[n])", "exp(-dl * Ad[n])")],
    "no_softplus": [("oracle_softplus(dr[t] + bias)", "(dr[t] + bias)")],
    "drop_delta_bias": [("oracle_softplus(dr[t] + bias)", "oracle_softplus(dr[t])")],
    "transposed_B_layout": [("dl * Bb[n * L + t] * ut", "dl * Bb[t * N + n] * ut")],
    "output_before_update": [(
        "h[n] = dA * h[n] + dBu;\n                acc += Cb[n * L + t] * h[n];",
        "acc += Cb[n * L + t] * h[n];\n                h[n] = dA * h[n] + dBu;")],
    "sigmoid_gate_not_silu": [("oracle_silu(zr[t])", "(1.0 / (1.0 + exp(-zr[t])))")],
    "input_term_without_delta": [("double dBu = dl * Bb[n * L + t] * ut;",
                                  "double dBu = Bb[n * L + t] * ut;")],
    "initial_state_ignored": [("h[n] = h0 ? h0[r * N + n] : 0.0;", "h[n] = 0.0;")],
    "C_index_shifted": [("acc += Cb[n * L + t] * h[n];",
                         "acc += Cb[n * L + (t > 0 ? t - 1 : 0)] * h[n];")],
    "decay_on_input_too": [("h[n] = dA * h[n] + dBu;", "h[n] = dA * (h[n] + dBu);")],
}

SSD_MUTANTS = {
    "identity": [],
    "ssd_no_softplus": [("oracle_softplus(dt[(b * L + t) * H + hh] + bias)",
                         "(dt[(b * L + t) * H + hh] + bias)")],
    "ssd_wrong_group": [("int64_t g = hh / heads_per_group;", "int64_t g = hh % G;")],
    "ssd_B_C_swapped": [("S[p * N + n] = a * S[p * N + n] + dx * Bt[n];",
                         "S[p * N + n] = a * S[p * N + n] + dx * Ct[n];")],
    "ssd_drop_skip": [("yt[p] = acc + skip * xt[p];", "yt[p] = acc;")],
    "ssd_decay_after_input": [("S[p * N + n] = a * S[p * N + n] + dx * Bt[n];",
                               "S[p * N + n] = a * (S[p * N + n] + dx * Bt[n]);")],
    "ssd_dt_index_wrong_head": [("dt[(b * L + t) * H + hh]", "dt[(b * L + t) * H + 0]")],
    "ssd_gate_ignored": [("if (zt) yt[p] *= oracle_silu(zt[p]);", "")],
    "ssd_sigmoid_gate_not_silu": [("if (zt) yt[p] *= oracle_silu(zt[p]);",
                                   "if (zt) yt[p] *= 1.0 / (1.0 + exp(-zt[p]));")],
    "ssd_gate_before_skip": [("yt[p] = acc + skip * xt[p];\n                if (zt) yt[p] *= oracle_silu(zt[p]);",
                              "yt[p] = (zt ? acc * oracle_silu(zt[p]) : acc) + skip * xt[p];")],
}


CONV_MUTANTS = {
    "identity": [],
    "conv_not_causal": [("int64_t s = t - (K - 1) + k;\n                if (s >= 0)",
                         "int64_t s = t + k;\n                if (s < L)")],
    "conv_taps_reversed": [("acc += w[k] * xr[s];", "acc += w[K - 1 - k] * xr[s];")],
    "conv_drop_bias": [("double bias = conv_b ? conv_b[d] : 0.0;", "double bias = 0.0;")],
    "conv_no_silu": [("u[r * L + t] = oracle_silu(acc);", "u[r * L + t] = acc;")],
}


def _build_variant(tmpdir, name, edits):
    src = open(ORACLE_C).read()
    for old, new in edits:
        assert old in src, "mutation anchor not found: %r" % old
        src = src.replace(old, new)
    c = os.path.join(tmpdir, name + ".c")
    so = os.path.join(tmpdir, name + ".so")
    with open(c, "w") as f:
        f.write(src)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared",
                    "-fPIC", "-std=c99", c, "-o", so, "-lm"], check=True)
    return oracle_py.load_variant(so)


def _scan_pins(lib):
    """The selective-scan pins, run against ``lib``; returns names that fail."""
    failed = []
    p = inputs.ScanProblem("m", 2, 21, 3, 4, "f32", "per_channel", True, True, 77)
    x = inputs.scan_inputs(p)
    h0 = np.random.default_rng(1).standard_normal((2, 3, 4))
    y, hl = oracle_py.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"],
                                     x["D"], x["z"], x["delta_bias"], h0=h0,
                                     lib=lib)
    yc, hc = pins.scan_closed_form(x["u"], x["delta"], x["A"], x["B"], x["C"],
                                   x["D"], x["z"], x["delta_bias"], h0=h0)
    if not (pins.rel_err(y, yc) < 1e-12 and pins.rel_err(hl, hc) < 1e-12):
        failed.append("closed_form")
    yl, hll = pins.scan_lifting(x["u"], x["delta"], x["A"], x["B"], x["C"],
                                x["D"], x["z"], x["delta_bias"])
    y0, h00 = oracle_py.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"],
                                       x["D"], x["z"], x["delta_bias"], lib=lib)
    if not (pins.rel_err(y0, yl) < 1e-12 and pins.rel_err(h00, hll) < 1e-12):
        failed.append("lifting")
    return failed


def _ssd_pins(lib):
    failed = []
    p = inputs.SSDProblem("m", 2, 40, 4, 3, 5, 2, "f32", 5)
    s = inputs.ssd_inputs(p)
    y, hl = oracle_py.ssd(s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"],
                          s["dt_bias"], lib=lib)
    yq = pins.ssd_quadratic(s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"], s["dt_bias"])
    if not pins.rel_err(y, yq, axis=1) < 1e-12:
        failed.append("quadratic")
    sg = inputs.ssd_inputs(p.replace(gate=True))
    yg, _ = oracle_py.ssd(sg["x"], sg["dt"], sg["A"], sg["B"], sg["C"], sg["D"],
                          sg["dt_bias"], z=sg["z"], lib=lib)
    yqg = pins.ssd_quadratic(sg["x"], sg["dt"], sg["A"], sg["B"], sg["C"], sg["D"],
                             sg["dt_bias"], z=sg["z"])
    if not pins.rel_err(yg, yqg, axis=1) < 1e-12:
        failed.append("gated_quadratic")
    yc, hc = pins.ssd_chunked(s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"],
                              s["dt_bias"], Q=16)
    if not (pins.rel_err(y, yc, axis=1) < 1e-12 and pins.rel_err(hl, hc) < 1e-12):
        failed.append("chunked")
    return failed


@pytest.mark.parametrize("name", sorted(SCAN_MUTANTS))
def test_scan_mutant_is_caught(tmp_path, name):
    lib = _build_variant(str(tmp_path), name, SCAN_MUTANTS[name])
    failed = _scan_pins(lib)
    if name == "identity":
        assert failed == []
    else:
        assert failed, "mutant %s passed every pin" % name


@pytest.mark.parametrize("name", sorted(SSD_MUTANTS))
def test_ssd_mutant_is_caught(tmp_path, name):
    lib = _build_variant(str(tmp_path), name, SSD_MUTANTS[name])
    failed = _ssd_pins(lib)
    if name == "identity":
        assert failed == []
    else:
        assert failed, "mutant %s passed every pin" % name


def _conv_pins(lib):
    import scipy.signal
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 3, 25))
    w = rng.standard_normal((3, 4))
    b = rng.standard_normal(3)
    u = oracle_py.conv1d_silu(x, w, b, lib=lib)
    ref = np.stack([[scipy.signal.lfilter(w[d, ::-1], [1.0], x[bb, d]) + b[d] for d in range(3)]
                    for bb in range(2)])
    return [] if pins.rel_err(u, pins.silu_lib(ref)) < 1e-14 else ["fir"]


@pytest.mark.parametrize("name", sorted(CONV_MUTANTS))
def test_conv_mutant_is_caught(tmp_path, name):
    lib = _build_variant(str(tmp_path), name, CONV_MUTANTS[name])
    failed = _conv_pins(lib)
    if name == "identity":
        assert failed == []
    else:
        assert failed, "mutant %s passed every pin" % name
