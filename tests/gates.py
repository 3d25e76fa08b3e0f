"""Parity gates between the GPU results and the float64 oracle.

The stated tolerance is a maximum relative error of 1e-4 for float32 I/O and
3e-3 for bfloat16 I/O, the oracle being fed the identical (bf16-rounded)
inputs.  Relative error of a single element is undefined where the output
crosses zero, and bf16 output rounding alone reaches 2^-8 = 3.9e-3 of an
element, so the gates read the tolerance this way:

  G1 (normwise, per row): max over rows r of ||got_r - ref_r||_2 / ||ref_r||_2
     <= tol, rows being (b, d) for the selective scan and (b, h, p) for SSD,
     against the UNROUNDED float64 oracle.  Applied to y and to h_last.
  G2 (elementwise): |got - ref| <= ulp_io(ref) + 1e-4 * max_t |ref_r|, which
     catches an isolated bad element that a norm would hide.

ulp_io is the spacing of the I/O format at |ref| (float32: 2^-23 relative,
bfloat16: 2^-7 relative, i.e. twice the worst rounding error).
"""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-4, "bf16": 3e-3}


def ulp(x, io):
    x = np.abs(np.asarray(x, np.float64))
    mant = 23 if io == "f32" else 7
    e = np.floor(np.log2(np.maximum(x, 1e-38)))
    return np.exp2(e - mant)


def g1(got, ref):
    """max over rows (last axis = the row's elements) of the 2-norm ratio."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.sqrt(np.sum((got - ref) ** 2, axis=-1))
    den = np.sqrt(np.sum(ref ** 2, axis=-1))
    den = np.where(den == 0, 1e-300, den)
    r = num / den
    return float(np.max(r)) if r.size else 0.0


def g2_worst(got, ref, io):
    """Largest ratio |err| / (ulp_io + 1e-4 * row max); <= 1 passes."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if not ref.size:
        return 0.0
    rowmax = np.max(np.abs(ref), axis=-1, keepdims=True)
    bound = ulp(ref, io) + 1e-4 * rowmax
    bound = np.where(bound == 0, 1e-300, bound)
    return float(np.max(np.abs(got - ref) / bound))


def check(got, ref, io, what=""):
    """Assert both gates; returns (g1, g2) for reporting."""
    assert np.all(np.isfinite(got)), "%s: non-finite values" % what
    e1 = g1(got, ref)
    e2 = g2_worst(got, ref, io)
    assert e1 <= TOL[io], "%s: G1 %.3e > %.1e" % (what, e1, TOL[io])
    assert e2 <= 1.0, "%s: G2 worst ratio %.3f > 1" % (what, e2)
    return e1, e2


def check_state(got, ref, io, what=""):
    """h_last is float32 whatever the I/O dtype: G1 at the I/O tolerance,
    G2 with float32 spacing (no output rounding is involved)."""
    assert np.all(np.isfinite(got)), "%s: non-finite values" % what
    e1 = g1(got, ref)
    e2 = g2_worst(got, ref, "f32")
    assert e1 <= TOL[io], "%s: G1 %.3e > %.1e" % (what, e1, TOL[io])
    assert e2 <= 1.0, "%s: G2 worst ratio %.3f > 1" % (what, e2)
    return e1, e2
