"""GPU parity of the selective scan fed by its convolution prologue
(mssm_selective_scan_fwd_conv) against the float64 oracle: the oracle's
causal width-4 convolution + SiLU, then its selective scan.  Needs an
MI355X; marked ``gpu``.
"""
from __future__ import annotations

import numpy as np
import pytest

import gates
from oracle import oracle
from selective_state_space_05_amd import _lib, inputs
from test_parity_gpu import announce, scan_to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SCAN_VARIANTS = [_lib.VARIANT_ROWSERIAL, _lib.VARIANT_CHUNKED, _lib.VARIANT_LOOKBACK]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def conv_to_dev(x, io, dev):
    t = scan_to_dev({k: v for k, v in x.items() if k not in ("conv_w", "conv_b")}, io, dev)
    t["conv_w"] = torch.from_numpy(x["conv_w"]).to(dev)
    t["conv_b"] = None if x["conv_b"] is None else torch.from_numpy(x["conv_b"]).to(dev)
    return t


def run_conv(t, variant, h0=None):
    import selective_state_space_05_amd as mssm
    from selective_state_space_05_amd.api import forced_variant
    with forced_variant(variant):
        y, h = mssm.selective_scan_conv_fwd(t["u"], t["conv_w"], t["delta"], t["A"], t["B"], t["C"],
                                            t["D"], t["z"], t["delta_bias"], conv_b=t["conv_b"],
                                            h0=h0)
    torch.cuda.synchronize()
    return f64(y), f64(h)


CONV_CASES = [
    # batch, L, dim, N, io, gate
    (2, 1000, 37, 16, "f32", True),          # ragged dim
    (2, 1000, 37, 16, "bf16", True),
    (1, 2, 9, 16, "f32", True),              # shorter than the window
    (1, 333, 20, 5, "bf16", False),          # odd L: element loads; N <= 8 layout
    (2, 4096 + 37, 40, 16, "bf16", True),    # several chunks and look-back segments
    (1, 2048, 24, 32, "f32", False),         # N <= 32 layout
    (1, 700, 17, 48, "bf16", True),          # N <= 64 layout
    (1, 8192, 16, 16, "bf16", False),        # vector loads across look-back segments
]


@pytest.mark.parametrize("variant", SCAN_VARIANTS)
@pytest.mark.parametrize("case", CONV_CASES)
def test_scan_with_conv_prologue(dev, variant, case):
    batch, L, dim, N, io, gate = case
    p = inputs.ScanProblem("case", batch, L, dim, N, io, "per_channel", gate, True, 400 + L + N,
                           conv=True)
    announce("scan conv variant=%d %s" % (variant, case))
    x = inputs.scan_inputs(p)
    y, h = run_conv(conv_to_dev(x, io, dev), variant)
    yo, ho = oracle.selective_scan_conv(x["u"], x["conv_w"], x["conv_b"], x["delta"], x["A"],
                                        x["B"], x["C"], x["D"], x["z"], x["delta_bias"])
    gates.check(y, yo, io, "y")
    gates.check_state(h, ho, io, "h_last")


@pytest.mark.parametrize("variant", SCAN_VARIANTS)
def test_scan_conv_without_bias_from_initial_state(dev, variant):
    p = inputs.ScanProblem("case", 2, 900, 33, 16, "bf16", "scalar", True, True, 61, conv=True)
    announce("scan conv no bias, h0, variant=%d" % variant)
    x = inputs.scan_inputs(p)
    x["conv_b"] = None
    h0 = inputs.initial_state((2, 33, 16), 9)
    y, h = run_conv(conv_to_dev(x, "bf16", dev), variant, h0=torch.from_numpy(h0).to(dev))
    yo, ho = oracle.selective_scan_conv(x["u"], x["conv_w"], None, x["delta"], x["A"], x["B"],
                                        x["C"], x["D"], x["z"], x["delta_bias"], h0=h0)
    gates.check(y, yo, "bf16", "y")
    gates.check_state(h, ho, "bf16", "h_last")


def test_scan_conv_full_size_sampled_rows(dev):
    """The Mamba-2.8B layer with the prologue, in the bench's launch
    configuration; rows are independent, so the oracle runs on a sample."""
    p = inputs.MAMBA_2_8B.replace(conv=True)
    announce("scan conv workload=%s" % p.name)
    x = inputs.scan_inputs(p)
    y, h = run_conv(conv_to_dev(x, p.io, dev), _lib.VARIANT_AUTO)
    rng = np.random.default_rng(4)
    rows = [(0, 0), (p.batch - 1, p.dim - 1)] + [
        (int(rng.integers(p.batch)), int(rng.integers(p.dim))) for _ in range(6)]
    for b, d in rows:
        sl = lambda a: None if a is None else a[b:b + 1, d:d + 1]   # noqa: E731
        pr = lambda a: None if a is None else a[d:d + 1]            # noqa: E731
        yo, ho = oracle.selective_scan_conv(sl(x["u"]), pr(x["conv_w"]), pr(x["conv_b"]),
                                            sl(x["delta"]), pr(x["A"]), x["B"][b:b + 1],
                                            x["C"][b:b + 1], pr(x["D"]), sl(x["z"]),
                                            pr(x["delta_bias"]))
        gates.check(y[b:b + 1, d], yo[:, 0], p.io, "y row (%d, %d)" % (b, d))
        gates.check_state(h[b:b + 1, d], ho[:, 0], p.io, "h_last row (%d, %d)" % (b, d))
