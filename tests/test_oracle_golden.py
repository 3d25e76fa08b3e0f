"""The float64 oracle against the 40-digit worked examples in tests/golden/.

The fixtures' citations name the definitions; their values come from
``tests/golden/make_golden.py``, which calls only the closed-form evaluator
in ``oracle/highprec.py`` (no recurrence is stepped there).
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _arr(v):
    return np.array(v, dtype=np.float64)


def _num(v):
    return np.vectorize(float)(np.array(v, dtype=object)).astype(np.float64)


def _close(got, ref, rtol=1e-14):
    """Elementwise |got - ref| <= rtol |ref|; exact zeros must be exact."""
    return bool(np.all(np.abs(got - ref) <= rtol * np.abs(ref)))


def test_scan_worked_example(oracle_mod):
    g = _load("scan_worked_example.json")
    assert g["citation"]
    y, hl = oracle_mod.selective_scan(_arr(g["u"]), _arr(g["delta"]), _arr(g["A"]),
                                      _arr(g["B"]), _arr(g["C"]), _arr(g["D"]),
                                      _arr(g["z"]), _arr(g["delta_bias"]))
    yr, hr = _num(g["y"]), _num(g["h_last"])
    assert _close(y, yr) and _close(hl, hr)


def test_ssd_worked_example(oracle_mod):
    g = _load("ssd_worked_example.json")
    assert g["citation"]
    y, _ = oracle_mod.ssd(_arr(g["x"]), _arr(g["dt"]), _arr(g["A"]), _arr(g["B"]),
                          _arr(g["C"]), _arr(g["D"]), _arr(g["dt_bias"]))
    yr = _num(g["y"])
    assert _close(y, yr)


def test_fixtures_regenerate_identically():
    """The stored digits are what the committed generator writes."""
    import sys
    sys.path.insert(0, GOLDEN)
    import make_golden
    from oracle import highprec
    g = _load("scan_worked_example.json")
    y, _ = highprec.selective_scan_closed_form(g["u"], g["delta"], g["A"], g["B"],
                                               g["C"], g["D"], g["z"], g["delta_bias"])
    assert [[make_golden._s(v) for v in row] for row in y[0]] == g["y"][0]
