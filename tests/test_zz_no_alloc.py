"""The entry point that allocates nothing (mssm_selective_scan_fwd_h0_noalloc)
against mssm_selective_scan_fwd_h0 on the same inputs: the same kernels, so
the outputs must be bitwise equal, and both within the parity gates of the
oracle.  Two calls in a row, the second with a smaller problem, so the
second runs on the scratch array the first left behind.  Needs an MI355X;
marked ``gpu``.
"""
from __future__ import annotations

import numpy as np
import pytest

import gates
from oracle import oracle
from selective_state_space_05_amd import _lib, inputs
from test_parity_gpu import announce, scan_problem, scan_to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _noalloc(t, h0, variant):
    import selective_state_space_05_amd as mssm
    from selective_state_space_05_amd.api import forced_variant
    y = torch.full_like(t["u"], float("nan"))
    h = torch.full((t["u"].shape[0], t["u"].shape[1], t["A"].shape[1]), float("nan"),
                   dtype=torch.float32, device=t["u"].device)
    with forced_variant(variant):
        mssm.selective_scan_fwd_noalloc(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                                        t["delta_bias"], h0, out=y, h_out=h)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), h.cpu().numpy().astype(np.float64)


def _allocating(t, h0, variant):
    import selective_state_space_05_amd as mssm
    from selective_state_space_05_amd.api import forced_variant
    with forced_variant(variant):
        y, h = mssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                                       t["delta_bias"], h0=h0)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), h.cpu().numpy().astype(np.float64)


# (batch, L, dim, N, io) of the first call, then of the smaller second call
PAIRS = [
    ((1, 20000 + 3, 40, 16, "bf16"), (1, 5000 + 1, 17, 16, "bf16")),
    ((2, 9000, 24, 32, "f32"), (1, 3000, 9, 7, "f32")),
]


@pytest.mark.parametrize("variant", [_lib.VARIANT_LOOKBACK, _lib.VARIANT_AUTO])
@pytest.mark.parametrize("pair", PAIRS)
def test_noalloc_matches_allocating_entry_point(dev, variant, pair):
    for i, (batch, L, dim, N, io) in enumerate(pair):
        p = scan_problem(batch, L, dim, N, io, 2000 + 17 * i + L, bias="per_channel")
        announce("no-alloc call %d variant=%d %s" % (i, variant, (batch, L, dim, N, io)))
        x = inputs.scan_inputs(p)
        t = scan_to_dev(x, io, dev)
        h0n = inputs.initial_state((batch, dim, N), 31 + i) if i == 1 else None
        h0 = None if h0n is None else torch.from_numpy(h0n).to(dev)
        yn, hn = _noalloc(t, h0, variant)
        ya, ha = _allocating(t, h0, variant)
        assert np.array_equal(yn, ya) and np.array_equal(hn, ha)
        yo, ho = oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"],
                                       x["z"], x["delta_bias"], h0=h0n)
        gates.check(yn, yo, io, "y")
        gates.check_state(hn, ho, io, "h_last")


def test_noalloc_million_step_sampled_rows(dev):
    """The million-step workload, which AUTO sends to the look-back variant,
    through the no-alloc entry point: sampled rows against the oracle."""
    p = inputs.MILLION
    announce("no-alloc workload=%s" % p.name)
    x = inputs.scan_inputs(p)
    t = scan_to_dev(x, p.io, dev)
    yn, hn = _noalloc(t, None, _lib.VARIANT_AUTO)
    rows = [(0, 0), (0, p.dim - 1), (0, 77), (0, 130)]
    yo, ho = oracle.selective_scan_rows(rows, x["u"], x["delta"], x["A"], x["B"], x["C"],
                                        x["D"], x["z"], x["delta_bias"])
    gates.check(np.stack([yn[b, d] for b, d in rows]), yo, p.io, "y")
    gates.check_state(np.stack([hn[b, d] for b, d in rows]), ho, p.io, "h_last")
