"""GPU parity of the entry points that carry a state between calls: both
forwards from an initial state h0, and the single decode step.  The float64
oracle takes the same h0 (its selective scan and SSD start from h0 when one
is given); a decode step is the oracle's selective scan over one time step
from the cached state.  Needs an MI355X; marked ``gpu``.
"""
from __future__ import annotations

import numpy as np
import pytest

import gates
from oracle import oracle
from selective_state_space_05_amd import _lib, inputs
from test_parity_gpu import announce, scan_to_dev, ssd_rows_of, ssd_to_dev, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SCAN_VARIANTS = [_lib.VARIANT_ROWSERIAL, _lib.VARIANT_CHUNKED, _lib.VARIANT_LOOKBACK]
SSD_VARIANTS = [_lib.VARIANT_SSD_RECURRENT, _lib.VARIANT_SSD_CHUNKED]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def scan_h0(t, h0, variant, h_out=None):
    import selective_state_space_05_amd as mssm
    from selective_state_space_05_amd.api import forced_variant
    with forced_variant(variant):
        y, h = mssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"],
                                       t["z"], t["delta_bias"], h0=h0, h_out=h_out)
    torch.cuda.synchronize()
    return y, h


SCAN_H0_CASES = [
    # batch, L, dim, N, io, bias, gate
    (2, 1000, 37, 16, "f32", "per_channel", True),
    (1, 4096 + 5, 40, 16, "bf16", "scalar", True),   # several look-back segments
    (2, 300, 9, 5, "bf16", None, False),              # odd N
    (1, 2500, 20, 48, "f32", "scalar", True),         # 32 < N <= 64
]


@pytest.mark.parametrize("variant", SCAN_VARIANTS)
@pytest.mark.parametrize("case", SCAN_H0_CASES)
def test_scan_from_initial_state(dev, variant, case):
    batch, L, dim, N, io, bias, gate = case
    p = inputs.ScanProblem("case", batch, L, dim, N, io, bias, gate, True, 300 + L + N)
    announce("scan h0 variant=%d %s" % (variant, case))
    x = inputs.scan_inputs(p)
    h0 = inputs.initial_state((batch, dim, N), 7 + N)
    y, h = scan_h0(scan_to_dev(x, io, dev), torch.from_numpy(h0).to(dev), variant)
    yo, ho = oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"],
                                   x["z"], x["delta_bias"], h0=h0)
    gates.check(f64(y), yo, io, "y")
    gates.check_state(f64(h), ho, io, "h_last")


@pytest.mark.parametrize("variant", SCAN_VARIANTS)
def test_scan_in_pieces_equals_whole(dev, variant):
    """A sequence cut in three pieces, each call continuing in place from the
    state the previous one left (h0 and h_out the same buffer), gives the
    whole sequence's outputs and final state."""
    p = inputs.ScanProblem("case", 2, 3000, 24, 16, "bf16", "scalar", True, True, 41)
    announce("scan in pieces variant=%d" % variant)
    x = inputs.scan_inputs(p)
    t = scan_to_dev(x, "bf16", dev)
    state = torch.zeros((2, 24, 16), dtype=torch.float32, device=dev)
    ys = []
    for a, b in ((0, 700), (700, 2048 + 700), (2048 + 700, 3000)):
        piece = dict(t)
        for k in ("u", "delta", "z", "B", "C"):
            piece[k] = t[k][..., a:b].contiguous()
        y, h = scan_h0(piece, state, variant, h_out=state)
        assert h.data_ptr() == state.data_ptr()
        ys.append(f64(y))
    yo, ho = oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"],
                                   x["z"], x["delta_bias"])
    gates.check(np.concatenate(ys, axis=-1), yo, "bf16", "y")
    gates.check_state(f64(state), ho, "bf16", "h_last")


SPLIT_CASES = [
    # batch, L, dim, N, io: every row group cut in two (few groups), and a
    # grid of 300 groups where the last 44 are cut (300 mod 256 compute units)
    (2, 2048 + 40, 40, 16, "bf16"),
    (1, 600, 16 * 300, 16, "f32"),
]


@pytest.mark.parametrize("case", SPLIT_CASES)
def test_scan_split_groups_equal_whole_walk(dev, case):
    """The chunked kernel cuts some row groups in two parts to balance the
    compute units, the second part recomputing the state at the cut with the
    state-only walk.  That is the same sequential evaluation, so the outputs
    must equal bit for bit those of the walk that keeps every group whole,
    which the kernel takes when h0 is the h_last buffer itself."""
    batch, L, dim, N, io = case
    p = inputs.ScanProblem("case", batch, L, dim, N, io, "scalar", True, True, 60 + N)
    announce("scan split vs whole %s" % (case,))
    x = inputs.scan_inputs(p)
    t = scan_to_dev(x, io, dev)
    h0 = torch.from_numpy(inputs.initial_state((batch, dim, N), 61)).to(dev)
    y_split, h_split = scan_h0(t, h0, _lib.VARIANT_CHUNKED)
    state = h0.clone()
    y_whole, h_whole = scan_h0(t, state, _lib.VARIANT_CHUNKED, h_out=state)
    assert torch.equal(y_split, y_whole)
    assert torch.equal(h_split, h_whole)


def test_scan_zero_length_copies_initial_state(dev):
    import selective_state_space_05_amd as mssm
    announce("scan h0 L=0")
    u = torch.empty((2, 3, 0), device=dev)
    A = -torch.ones((3, 4), device=dev)
    B = torch.empty((2, 4, 0), device=dev)
    h0 = torch.randn((2, 3, 4), device=dev)
    _, h = mssm.selective_scan_fwd(u, u.clone(), A, B, B.clone(), h0=h0)
    torch.cuda.synchronize()
    assert torch.equal(h, h0)


SSD_H0_CASES = [
    # batch, L, H, P, N, G, io
    (1, 300, 2, 8, 16, 1, "bf16"),
    (2, 513, 4, 64, 128, 1, "bf16"),
    (1, 1000, 3, 40, 7, 3, "bf16"),
    (1, 77, 6, 5, 7, 3, "f32"),
]


@pytest.mark.parametrize("variant", SSD_VARIANTS)
@pytest.mark.parametrize("case", SSD_H0_CASES)
def test_ssd_from_initial_state(dev, variant, case):
    import selective_state_space_05_amd as mssm
    from selective_state_space_05_amd.api import forced_variant
    batch, L, H, P, N, G, io = case
    if variant == _lib.VARIANT_SSD_CHUNKED and io != "bf16":
        pytest.skip("the matrix-core form takes bf16 activations only")
    announce("ssd h0 variant=%d %s" % (variant, case))
    p = inputs.SSDProblem("case", batch, L, H, P, N, G, io, 900 + L)
    s = inputs.ssd_inputs(p)
    h0 = inputs.initial_state((batch, H, P, N), 11 + N)
    t = ssd_to_dev(s, io, dev)
    with forced_variant(variant):
        y, h = mssm.ssd_scalar_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"],
                                   t["dt_bias"], h0=torch.from_numpy(h0).to(dev))
    torch.cuda.synchronize()
    yo, ho = oracle.ssd(s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"], s["dt_bias"], h0=h0)
    gates.check(ssd_rows_of(f64(y)), ssd_rows_of(yo), io, "y")
    gates.check_state(f64(h), ho, io, "h_last")


@pytest.mark.parametrize("variant", SSD_VARIANTS)
def test_ssd_in_pieces_equals_whole(dev, variant):
    import selective_state_space_05_amd as mssm
    from selective_state_space_05_amd.api import forced_variant
    p = inputs.SSDProblem("case", 2, 1300, 4, 32, 64, 2, "bf16", 57)
    announce("ssd in pieces variant=%d" % variant)
    s = inputs.ssd_inputs(p)
    t = ssd_to_dev(s, "bf16", dev)
    state = torch.zeros((2, 4, 32, 64), dtype=torch.float32, device=dev)
    ys = []
    with forced_variant(variant):
        for a, b in ((0, 600), (600, 1300)):
            piece = {k: (v[:, a:b].contiguous() if k in ("x", "dt", "B", "C") else v)
                     for k, v in t.items()}
            y, _ = mssm.ssd_scalar_fwd(piece["x"], piece["dt"], piece["A"], piece["B"],
                                       piece["C"], piece["D"], piece["dt_bias"], h0=state,
                                       h_out=state)
            ys.append(f64(y))
    torch.cuda.synchronize()
    yo, ho = oracle.ssd(s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"], s["dt_bias"])
    gates.check(ssd_rows_of(np.concatenate(ys, axis=1)), ssd_rows_of(yo), "bf16", "y")
    gates.check_state(f64(state), ho, "bf16", "h_last")


# ---------------------------------------------------------------------------
# SSD with a SiLU gate on the output
# ---------------------------------------------------------------------------
SSD_GATED_CASES = [
    # batch, L, H, P, N, G, io, with h0
    (1, 300, 2, 8, 16, 1, "bf16", False),
    (2, 513, 4, 64, 128, 1, "bf16", True),    # three chunks, ragged, from h0
    (1, 1000, 3, 40, 7, 3, "bf16", False),    # two head-dim tiles, element path
    (1, 600, 2, 80, 96, 1, "bf16", True),     # two 64-column head-dim slices
    (1, 77, 6, 5, 7, 3, "f32", True),
    (1, 700, 3, 64, 64, 1, "bf16", True),     # odd head count per group, from h0
]


@pytest.mark.parametrize("variant", SSD_VARIANTS)
@pytest.mark.parametrize("case", SSD_GATED_CASES)
def test_ssd_gated(dev, variant, case):
    import selective_state_space_05_amd as mssm
    from selective_state_space_05_amd.api import forced_variant
    batch, L, H, P, N, G, io, with_h0 = case
    if variant == _lib.VARIANT_SSD_CHUNKED and io != "bf16":
        pytest.skip("the matrix-core form takes bf16 activations only")
    announce("ssd gated variant=%d %s" % (variant, case))
    p = inputs.SSDProblem("case", batch, L, H, P, N, G, io, 700 + L, gate=True)
    s = inputs.ssd_inputs(p)
    h0 = inputs.initial_state((batch, H, P, N), 5 + N) if with_h0 else None
    t = ssd_to_dev(s, io, dev)
    with forced_variant(variant):
        y, h = mssm.ssd_scalar_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"],
                                   t["dt_bias"], z=t["z"],
                                   h0=None if h0 is None else torch.from_numpy(h0).to(dev))
    torch.cuda.synchronize()
    yo, ho = oracle.ssd(s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"], s["dt_bias"],
                        h0=h0, z=s["z"])
    gates.check(ssd_rows_of(f64(y)), ssd_rows_of(yo), io, "y")
    gates.check_state(f64(h), ho, io, "h_last")


def test_ssd_gated_full_size_sampled_rows(dev):
    """The Mamba-2 layer with a gate, in the bench's launch configuration."""
    import selective_state_space_05_amd as mssm
    p = inputs.SSD_LAYER.replace(gate=True)
    announce("ssd gated workload=%s" % p.name)
    s = inputs.ssd_inputs(p)
    t = ssd_to_dev(s, p.io, dev)
    y, h = mssm.ssd_scalar_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["dt_bias"],
                               z=t["z"])
    torch.cuda.synchronize()
    y, h = f64(y), f64(h)
    rng = np.random.default_rng(8)
    rows = [(0, 0, 0), (p.batch - 1, p.nheads - 1, p.headdim - 1)] + [
        (int(rng.integers(p.batch)), int(rng.integers(p.nheads)), int(rng.integers(p.headdim)))
        for _ in range(6)]
    yo, ho = oracle.ssd_rows(rows, s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"],
                             s["dt_bias"], z=s["z"])
    gates.check(np.stack([y[b, :, hh, pp] for b, hh, pp in rows]), yo, p.io, "y")
    gates.check_state(np.stack([h[b, hh, pp] for b, hh, pp in rows]), ho, p.io, "h_last")


# Many heads (grids of 768 and more workgroups) with ragged chunk counts:
# the output workgroups walk chunk pairs, the last pair without a partner
# where the count is odd; sampled rows, with a gate and from h0.
SSD_WIDE_CASES = [
    # batch, L, H, P, N, G, gate, with h0
    (1, 1300, 384, 64, 64, 4, False, False),   # 6 chunks
    (2, 1700, 192, 64, 128, 2, True, True),    # 7 chunks: a chunk without a partner
    (1, 1025, 384, 80, 32, 1, False, True),    # 5 chunks; two head-dim slices
]


@pytest.mark.parametrize("case", SSD_WIDE_CASES)
def test_ssd_wide_grid_sampled_rows(dev, case):
    import selective_state_space_05_amd as mssm
    from selective_state_space_05_amd.api import forced_variant
    batch, L, H, P, N, G, gate, with_h0 = case
    announce("ssd wide grid %s" % (case,))
    p = inputs.SSDProblem("case", batch, L, H, P, N, G, "bf16", 400 + L, gate=gate)
    s = inputs.ssd_inputs(p)
    h0 = inputs.initial_state((batch, H, P, N), 3 + N) if with_h0 else None
    t = ssd_to_dev(s, "bf16", dev)
    with forced_variant(_lib.VARIANT_SSD_CHUNKED):
        y, h = mssm.ssd_scalar_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"],
                                   t["dt_bias"], z=t["z"] if gate else None,
                                   h0=None if h0 is None else torch.from_numpy(h0).to(dev))
    torch.cuda.synchronize()
    y, h = f64(y), f64(h)
    rng = np.random.default_rng(L)
    rows = [(0, 0, 0), (batch - 1, H - 1, P - 1)] + [
        (int(rng.integers(batch)), int(rng.integers(H)), int(rng.integers(P))) for _ in range(8)]
    yo, ho = oracle.ssd_rows(rows, s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"],
                             s["dt_bias"], z=s["z"] if gate else None, h0=h0)
    gates.check(np.stack([y[b, :, hh, pp] for b, hh, pp in rows]), yo, "bf16", "y")
    gates.check_state(np.stack([h[b, hh, pp] for b, hh, pp in rows]), ho, "bf16", "h_last")


# ---------------------------------------------------------------------------
# decode step
# ---------------------------------------------------------------------------
def step_to_dev(d, io, dev, offset=0):
    """Device copies of one step's operands.  offset > 0 places every
    activation and the state one element past an aligned start, which sends
    the kernel down its scalar-load path."""
    out = {}
    for k, v in d.items():
        if v is None:
            out[k] = None
        elif k in ("A", "D", "dt_bias", "state"):
            t = torch.from_numpy(np.ascontiguousarray(v))
            if k == "state" and offset:
                buf = torch.empty(t.numel() + offset, dtype=torch.float32)
                buf[offset:] = t.reshape(-1)
                out[k] = buf.to(dev)[offset:].view(v.shape)
            else:
                out[k] = t.to(dev)
        else:
            t = to_dev(v, io, dev)
            if offset:
                buf = torch.empty(t.numel() + offset, dtype=t.dtype, device=dev)
                buf[offset:] = t.reshape(-1)
                t = buf[offset:].view(v.shape)
            out[k] = t
    return out


def run_step(t):
    import selective_state_space_05_amd as mssm
    y = mssm.selective_state_update(t["state"], t["x"], t["dt"], t["A"], t["B"], t["C"],
                                    t["D"], t["z"], t["dt_bias"])
    torch.cuda.synchronize()
    return f64(y), t["state"].cpu().numpy().astype(np.float64)


def step_oracle(d):
    """The oracle's scan over the single time step, from the cached state."""
    col = lambda a: None if a is None else a[..., None]   # noqa: E731
    yo, ho = oracle.selective_scan(col(d["x"]), col(d["dt"]), d["A"], col(d["B"]),
                                   col(d["C"]), d["D"], col(d["z"]), d["dt_bias"],
                                   h0=d["state"])
    return yo[..., 0], ho


STEP_CASES = [
    # batch, dim, N, io, bias, gate, skip, offset
    (3, 37, 16, "f32", "per_channel", True, True, 0),
    (3, 37, 16, "bf16", "scalar", True, True, 0),
    (2, 130, 4, "bf16", None, False, True, 0),      # one lane per row
    (2, 50, 1, "f32", "scalar", True, False, 0),    # N = 1
    (1, 70, 7, "bf16", "scalar", True, True, 0),    # N % 4 != 0: scalar loads
    (2, 33, 64, "f32", "per_channel", True, True, 0),   # 16 lanes per row
    (2, 45, 36, "bf16", "scalar", False, True, 0),  # 9 quads in 16 lanes
    (2, 40, 16, "bf16", "scalar", True, True, 1),   # misaligned operands
    (1, 1, 16, "f32", "scalar", True, True, 0),     # a single row
]


@pytest.mark.parametrize("case", STEP_CASES)
def test_step_small_full_compare(dev, case):
    batch, dim, N, io, bias, gate, skip, offset = case
    p = inputs.StepProblem("case", batch, dim, N, io, bias, gate, skip, 500 + dim + N)
    announce("step %s" % (case,))
    d = inputs.step_inputs(p)
    y, h = run_step(step_to_dev(d, io, dev, offset))
    yo, ho = step_oracle(d)
    # normwise rows are a sequence's outputs over the channels, y[b, :] (a
    # (b, d) row of one step is a single bf16-rounded element); the
    # elementwise gate still checks every output
    gates.check(y, yo, io, "y")
    # the state's normwise rows are likewise one sequence's whole state
    gates.check_state(h.reshape(batch, -1), ho.reshape(batch, -1), io, "state")


def test_step_repeated_equals_scan(dev):
    """T decode steps on one state reproduce the scan over those T steps."""
    p = inputs.ScanProblem("case", 2, 40, 24, 16, "bf16", "scalar", True, True, 77)
    announce("step repeated")
    x = inputs.scan_inputs(p)
    h0 = inputs.initial_state((2, 24, 16), 3)
    t = scan_to_dev(x, "bf16", dev)
    state = torch.from_numpy(h0).to(dev)
    import selective_state_space_05_amd as mssm
    ys = []
    for s in range(p.seqlen):
        step = {k: t[k][..., s].contiguous() for k in ("u", "delta", "B", "C", "z")}
        ys.append(f64(mssm.selective_state_update(state, step["u"], step["delta"], t["A"],
                                                  step["B"], step["C"], t["D"], step["z"],
                                                  t["delta_bias"])))
    torch.cuda.synchronize()
    yo, ho = oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"],
                                   x["z"], x["delta_bias"], h0=h0)
    gates.check(np.stack(ys, axis=-1), yo, "bf16", "y")
    gates.check_state(state.cpu().numpy().astype(np.float64), ho, "bf16", "state")


def test_step_full_size(dev):
    """The decode workload the benchmark times, compared over every row."""
    p = inputs.DECODE_2_8B
    announce("step workload=%s" % p.name)
    d = inputs.step_inputs(p)
    y, h = run_step(step_to_dev(d, p.io, dev))
    yo, ho = step_oracle(d)
    gates.check(y.reshape(p.batch, -1), yo.reshape(p.batch, -1), p.io, "y")
    rng = np.random.default_rng(0)
    rows = rng.integers(0, p.batch, 64)
    gates.check_state(h[rows].reshape(64, -1), ho[rows].reshape(64, -1), p.io, "state")
    assert np.all(np.isfinite(h))
