"""Write the worked-example fixtures in this directory.

Calls only ``oracle/`` (the 40-digit closed-form evaluator in
``oracle/highprec.py``).  The pages print no numeric example for the scan,
so these fixtures are tiny hand-chosen problems whose inputs are dyadic
rationals (exact in float32 and float64) and whose outputs are the closed
form evaluated at 40 significant digits, stored to 30.

Run from the repository root:  python tests/golden/make_golden.py
"""
from __future__ import annotations

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import highprec  # noqa: E402

SCAN = {
    "citation": (
        "Selective-scan definition: 'Mamba状态空间模型的硬件感知推理优化' "
        "(ybb.press) sections 1 and 3.1 (recurrence, decay exp(A*softplus(dt)), "
        "y = C.h + D*x); www.mhpq.cn/news/984979 essay sections 2.2-2.3 (ZOH "
        "step, unrolled closed form); '从硬件感知到算法革命' (tencentcloud.csdn.net) "
        "sections 2-3 (softplus step size, SiLU gate).  Values: closed form at "
        "40 digits; the pages print no numeric example."),
    "u": [[[0.5, -1.25, 2.0, 0.125, -0.75], [1.5, 0.25, -0.5, -2.0, 1.0]]],
    "delta": [[[-2.0, -1.5, -2.5, -1.0, -3.0], [-1.75, -2.25, -0.5, -2.0, -1.25]]],
    "delta_bias": [0.5, -0.25],
    "A": [[-1.0, -3.5, -8.0], [-2.0, -0.5, -6.25]],
    "B": [[[1.0, -0.5, 0.25, 2.0, -1.5], [0.75, 1.25, -2.0, 0.5, 0.0],
           [-1.0, 0.375, 1.5, -0.25, 1.0]]],
    "C": [[[0.5, 1.0, -1.5, 0.25, 2.0], [-0.25, 0.75, 1.0, -1.0, 0.5],
           [1.5, -0.5, 0.125, 1.25, -2.0]]],
    "D": [0.625, -1.125],
    "z": [[[1.0, -0.5, 2.5, -2.0, 0.25], [0.0, 1.5, -1.0, 3.0, -0.125]]],
}

SSD = {
    "citation": (
        "Mamba-2 scalar decay: 'Mamba状态空间模型的硬件感知推理优化' (ybb.press) "
        "section 4 (per-step scalar decay, cumulative-product form) and section "
        "6.2 (log-space products).  Values: quadratic form at 40 digits."),
    "x": [[[[0.5, -1.0], [1.25, 0.25]], [[-0.75, 2.0], [0.5, -1.5]],
           [[1.0, 0.125], [-2.0, 0.75]], [[0.25, -0.5], [1.5, 1.0]]]],
    "dt": [[[-2.0, -1.5], [-2.5, -1.0], [-1.75, -3.0], [-0.5, -2.25]]],
    "dt_bias": [-3.0, -2.5],
    "A": [-1.5, -7.0],
    "B": [[[[1.0, -0.5, 0.25]], [[2.0, 0.75, -1.0]], [[-1.5, 0.5, 1.25]],
           [[0.0, -2.0, 0.375]]]],
    "C": [[[[0.5, 1.5, -1.0]], [[-0.25, 1.0, 0.5]], [[1.0, -0.75, 2.0]],
           [[1.25, 0.25, -0.5]]]],
    "D": [0.75, -1.25],
}


def _s(v):
    return highprec.mpmath.nstr(v, 30, strip_zeros=False)


def main():
    y, hl = highprec.selective_scan_closed_form(
        SCAN["u"], SCAN["delta"], SCAN["A"], SCAN["B"], SCAN["C"], SCAN["D"],
        SCAN["z"], SCAN["delta_bias"])
    out = dict(SCAN)
    out["y"] = [[[_s(v) for v in row] for row in b] for b in y]
    out["h_last"] = [[[_s(v) for v in row] for row in b] for b in hl]
    with open(os.path.join(HERE, "scan_worked_example.json"), "w") as f:
        json.dump(out, f, indent=1, ensure_ascii=False)
        f.write("\n")

    ys = highprec.ssd_closed_form(SSD["x"], SSD["dt"], SSD["A"], SSD["B"],
                                  SSD["C"], SSD["D"], SSD["dt_bias"])
    out = dict(SSD)
    out["y"] = [[[[_s(v) for v in hp] for hp in t] for t in b] for b in ys]
    with open(os.path.join(HERE, "ssd_worked_example.json"), "w") as f:
        json.dump(out, f, indent=1, ensure_ascii=False)
        f.write("\n")


if __name__ == "__main__":
    main()
