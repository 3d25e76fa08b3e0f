"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
identical seeded inputs.  Needs an MI355X; marked ``gpu``.

Small problems are compared element by element over the whole output; the
full-size workloads run in the same launch configuration the benchmark
times and are compared on sampled rows, which the oracle computes exactly
as in the full problem because rows are independent.
"""
from __future__ import annotations

import numpy as np
import pytest

import gates
from oracle import oracle
from selective_state_space_05_amd import _lib, inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SCAN_VARIANTS = [_lib.VARIANT_ROWSERIAL, _lib.VARIANT_CHUNKED, _lib.VARIANT_LOOKBACK]
SSD_VARIANTS = [_lib.VARIANT_SSD_RECURRENT, _lib.VARIANT_SSD_CHUNKED]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(a, io, dev):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if io == "bf16" and a.ndim > 1:
        t = t.to(torch.bfloat16)     # exact: values are already bf16
    return t.to(dev)


def scan_to_dev(x, io, dev):
    out = {}
    for k, v in x.items():
        if k in ("A", "D", "delta_bias"):
            out[k] = None if v is None else torch.from_numpy(v).to(dev)
        else:
            out[k] = to_dev(v, io, dev)
    return out


def run_scan(t, variant=_lib.VARIANT_AUTO, stream=None):
    import selective_state_space_05_amd as mssm
    from selective_state_space_05_amd.api import forced_variant
    with forced_variant(variant):
        if stream is None:
            y, h = mssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"],
                                           t["D"], t["z"], t["delta_bias"])
        else:
            with torch.cuda.stream(stream):
                y, h = mssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"],
                                               t["C"], t["D"], t["z"], t["delta_bias"])
            stream.synchronize()
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), h.cpu().numpy().astype(np.float64)


def scan_problem(batch, L, dim, N, io, seed, bias="scalar", gate=True, skip=True):
    return inputs.ScanProblem("case", batch, L, dim, N, io, bias, gate, skip, seed)


def announce(msg):
    print("\n[gpu case] %s" % msg, flush=True)


SMALL_CASES = [
    # batch, L, dim, N, io, bias, gate, skip
    (1, 64, 8, 4, "f32", "scalar", False, True),          # the tiny workload
    (2, 1000, 37, 16, "f32", "per_channel", True, True),   # ragged L and dim
    (2, 1000, 37, 16, "bf16", "scalar", True, True),
    (1, 1, 5, 16, "f32", "scalar", True, True),            # single step
    (3, 7, 3, 1, "f32", None, False, False),               # N = 1, no extras
    (1, 333, 64, 5, "bf16", "per_channel", False, True),   # odd N
    (2, 4096 + 37, 40, 16, "bf16", "scalar", True, True),  # several chunks
    (1, 2048, 130, 32, "f32", "scalar", True, True),       # N = 32
    (1, 300, 9, 64, "f32", "scalar", True, True),          # N = 64 (limit)
    (2, 2500 + 5, 20, 48, "bf16", "per_channel", True, True),  # 32 < N < 64, several chunks
    (1, 20000 + 3, 17, 16, "bf16", "per_channel", True, True),  # many segments, ragged
    (3, 6000, 8, 7, "f32", "scalar", False, True),         # N = 7, three batches
]


@pytest.mark.parametrize("variant", SCAN_VARIANTS)
@pytest.mark.parametrize("case", SMALL_CASES)
def test_scan_small_full_compare(dev, variant, case):
    batch, L, dim, N, io, bias, gate, skip = case
    p = scan_problem(batch, L, dim, N, io, 1000 + L + dim, bias, gate, skip)
    announce("scan variant=%d %s" % (variant, case))
    x = inputs.scan_inputs(p)
    y, h = run_scan(scan_to_dev(x, io, dev), variant)
    yo, ho = oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"],
                                   x["D"], x["z"], x["delta_bias"])
    gates.check(y, yo, io, "y")
    gates.check_state(h, ho, io, "h_last")


def _sampled(p, variant, dev, nrows=12, seed=0):
    x = inputs.scan_inputs(p)
    announce("scan variant=%d workload=%s" % (variant, p.name))
    y, h = run_scan(scan_to_dev(x, p.io, dev), variant)
    rng = np.random.default_rng(seed)
    rows = [(0, 0), (p.batch - 1, p.dim - 1)] + [
        (int(rng.integers(p.batch)), int(rng.integers(p.dim))) for _ in range(nrows - 2)]
    yo, ho = oracle.selective_scan_rows(rows, x["u"], x["delta"], x["A"], x["B"], x["C"],
                                        x["D"], x["z"], x["delta_bias"])
    ys = np.stack([y[b, d] for b, d in rows])
    hs = np.stack([h[b, d] for b, d in rows])
    gates.check(ys, yo, p.io, "y %s" % p.name)
    gates.check_state(hs, ho, p.io, "h_last %s" % p.name)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(h))


@pytest.mark.parametrize("variant", [_lib.VARIANT_AUTO] + SCAN_VARIANTS)
def test_scan_tiny_workload_as_stated(dev, variant):
    """The tiny workload exactly as stated: batch 1, L 64, 8 channels, N 4,
    float32, seed 0, bias 0.5, skip term, no gate, h0 = 0; every element of
    y and h_last against the oracle (which the CPU tests pin to the
    brute-force closed form on these very inputs)."""
    p = inputs.TINY
    assert (p.seed, p.gate, p.skip, p.bias, p.io) == (0, False, True, "scalar", "f32")
    announce("scan variant=%d workload=%s" % (variant, p.name))
    x = inputs.scan_inputs(p)
    assert x["z"] is None
    y, h = run_scan(scan_to_dev(x, p.io, dev), variant)
    yo, ho = oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"],
                                   x["D"], x["z"], x["delta_bias"])
    gates.check(y, yo, p.io, "y")
    gates.check_state(h, ho, p.io, "h_last")


PAIR_VARIANTS = [_lib.VARIANT_PAIRSCAN, _lib.VARIANT_PAIRSCAN2]


@pytest.mark.parametrize("variant", PAIR_VARIANTS)
@pytest.mark.parametrize("case", [c for c in SMALL_CASES if c[3] <= 16] + [
    (2, 64 * 5 + 64, 16, 16, "f32", "per_channel", True, True),   # whole chunks only
    (1, 64 * 3 + 17, 48, 16, "bf16", "scalar", True, True),       # three channel groups, tail
    (1, 1000, 16, 9, "f32", "scalar", False, False),              # no optional inputs
])
def test_scan_pairscan_small_full_compare(dev, variant, case):
    """The pair-scan variants (steps of each chunk split across lanes) on
    every small case they support (N <= 16), element by element."""
    batch, L, dim, N, io, bias, gate, skip = case
    p = scan_problem(batch, L, dim, N, io, 1000 + L + dim, bias, gate, skip)
    announce("scan variant=%d %s" % (variant, case))
    x = inputs.scan_inputs(p)
    y, h = run_scan(scan_to_dev(x, io, dev), variant)
    yo, ho = oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"],
                                   x["D"], x["z"], x["delta_bias"])
    gates.check(y, yo, io, "y")
    gates.check_state(h, ho, io, "h_last")


@pytest.mark.parametrize("variant", PAIR_VARIANTS)
def test_scan_pairscan_from_initial_state(dev, variant):
    p = scan_problem(2, 777, 24, 16, "bf16", 71, bias="per_channel")
    announce("scan variant=%d from h0" % variant)
    x = inputs.scan_inputs(p)
    h0 = inputs.initial_state((2, 24, 16), 72)
    t = scan_to_dev(x, "bf16", dev)
    import selective_state_space_05_amd as mssm
    from selective_state_space_05_amd.api import forced_variant
    with forced_variant(variant):
        y, h = mssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                                       t["delta_bias"], h0=torch.from_numpy(h0).to(dev))
    torch.cuda.synchronize()
    yo, ho = oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"],
                                   x["delta_bias"], h0=h0)
    gates.check(y.float().cpu().numpy().astype(np.float64), yo, "bf16", "y")
    gates.check_state(h.cpu().numpy().astype(np.float64), ho, "bf16", "h_last")


@pytest.mark.parametrize("variant", PAIR_VARIANTS)
def test_scan_pairscan_deterministic(dev, variant):
    p = scan_problem(2, 3000, 40, 16, "bf16", 73)
    t = scan_to_dev(inputs.scan_inputs(p), "bf16", dev)
    announce("scan variant=%d determinism" % variant)
    y1, h1 = run_scan(t, variant)
    y2, h2 = run_scan(t, variant)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


def test_scan_pairscan_rejects_large_state(dev):
    import selective_state_space_05_amd as mssm
    from selective_state_space_05_amd.api import MssmError, forced_variant
    p = scan_problem(1, 256, 16, 32, "f32", 74)
    t = scan_to_dev(inputs.scan_inputs(p), "f32", dev)
    with forced_variant(_lib.VARIANT_PAIRSCAN):
        with pytest.raises(MssmError):
            mssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"])


FULL = [inputs.MAMBA_130M, inputs.MAMBA_2_8B, inputs.MILLION]
# AUTO's kernel on each layer shape: the look-back kernel where the chunked
# grid fills under four fifths of the 1024 SIMDs and the rows are long
AUTO_CHOICE = {inputs.MAMBA_130M.name: _lib.VARIANT_LOOKBACK,
               inputs.MAMBA_2_8B.name: _lib.VARIANT_CHUNKED,
               inputs.MILLION.name: _lib.VARIANT_LOOKBACK}


@pytest.mark.parametrize("variant", [_lib.VARIANT_AUTO] + SCAN_VARIANTS + PAIR_VARIANTS)
@pytest.mark.parametrize("p", FULL, ids=[q.name for q in FULL])
def test_scan_full_size_sampled_rows(dev, variant, p):
    from selective_state_space_05_amd.api import last_variant
    _sampled(p, variant, dev)
    assert last_variant() == (AUTO_CHOICE[p.name] if variant == _lib.VARIANT_AUTO else variant)


@pytest.mark.parametrize("p", FULL, ids=[q.name for q in FULL])
def test_scan_full_size_scan_isolated(dev, p):
    """No skip term and no gate: y = C.h exactly, so the scan's own error is
    not hidden behind D*u."""
    _sampled(p.replace(skip=False, gate=False), _lib.VARIANT_AUTO, dev, nrows=8, seed=1)


@pytest.mark.parametrize("p", [inputs.MAMBA_2_8B, inputs.MILLION],
                         ids=["mamba2.8b", "million"])
def test_scan_full_size_per_channel_bias(dev, p):
    """The other reading of the bias distribution (per channel U(-4, -2))."""
    _sampled(p.replace(bias="per_channel"), _lib.VARIANT_AUTO, dev, nrows=8, seed=2)


def test_scan_deterministic(dev):
    p = scan_problem(2, 3000, 64, 16, "bf16", 5)
    t = scan_to_dev(inputs.scan_inputs(p), "bf16", dev)
    announce("scan determinism")
    y1, h1 = run_scan(t)
    y2, h2 = run_scan(t)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


def test_scan_on_side_stream(dev):
    p = scan_problem(2, 500, 33, 16, "f32", 6)
    x = inputs.scan_inputs(p)
    t = scan_to_dev(x, "f32", dev)
    announce("scan side stream")
    s = torch.cuda.Stream(dev)
    y, h = run_scan(t, stream=s)
    yo, ho = oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"],
                                   x["z"], x["delta_bias"])
    gates.check(y, yo, "f32", "y")
    gates.check_state(h, ho, "f32", "h_last")


def test_scan_zero_length_zero_fills_state(dev):
    import selective_state_space_05_amd as mssm
    announce("scan L=0")
    u = torch.empty((2, 3, 0), device=dev)
    A = -torch.ones((3, 4), device=dev)
    B = torch.empty((2, 4, 0), device=dev)
    h_out = torch.full((2, 3, 4), 7.0, device=dev)
    y, h = mssm.selective_scan_fwd(u, u.clone(), A, B, B.clone(), h_out=h_out)
    torch.cuda.synchronize()
    assert y.shape == (2, 3, 0) and torch.all(h == 0)


def test_scan_auto_picks_lookback_for_few_long_rows(dev):
    from selective_state_space_05_amd.api import last_variant
    p = scan_problem(1, 8192, 32, 16, "bf16", 8)
    announce("scan auto look-back")
    x = inputs.scan_inputs(p)
    y, h = run_scan(scan_to_dev(x, "bf16", dev))
    assert last_variant() == _lib.VARIANT_LOOKBACK
    yo, ho = oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"],
                                   x["z"], x["delta_bias"])
    gates.check(y, yo, "bf16", "y")
    gates.check_state(h, ho, "bf16", "h_last")


def test_scan_lookback_deterministic(dev):
    p = scan_problem(1, 50000, 16, 16, "f32", 9, bias="per_channel")
    t = scan_to_dev(inputs.scan_inputs(p), "f32", dev)
    announce("scan look-back determinism")
    y1, h1 = run_scan(t, _lib.VARIANT_LOOKBACK)
    y2, h2 = run_scan(t, _lib.VARIANT_LOOKBACK)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


def test_scan_reports_variant(dev):
    from selective_state_space_05_amd.api import last_variant
    p = scan_problem(1, 64, 8, 4, "f32", 7)
    run_scan(scan_to_dev(inputs.scan_inputs(p), "f32", dev))
    assert last_variant() != _lib.VARIANT_AUTO


# ---------------------------------------------------------------------------
# SSD
# ---------------------------------------------------------------------------
def ssd_to_dev(s, io, dev):
    out = {}
    for k, v in s.items():
        if k in ("A", "D", "dt_bias"):
            out[k] = None if v is None else torch.from_numpy(v).to(dev)
        else:
            out[k] = to_dev(v, io, dev)
    return out


def run_ssd(t, variant=_lib.VARIANT_AUTO, chunk=0):
    import selective_state_space_05_amd as mssm
    from selective_state_space_05_amd.api import forced_variant
    with forced_variant(variant):
        y, h = mssm.ssd_scalar_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"],
                                   t["dt_bias"], chunk=chunk)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), h.cpu().numpy().astype(np.float64)


def ssd_rows_of(y):
    """(batch, L, H, P) -> the rows of the normwise gate.

    A row is one (b, h, p) sequence of L outputs.  With L = 1 such a row is
    a single bf16-rounded element, whose rounding alone can exceed the
    tolerance, so there a head's whole block (batch, H) of P outputs is one
    row."""
    b, L, H, P = y.shape
    if L == 1:
        return np.ascontiguousarray(np.moveaxis(y, 2, 1)).reshape(b, H, L * P)
    return np.ascontiguousarray(np.transpose(y, (0, 2, 3, 1)))   # (b, H, P, L)


SSD_SMALL = [
    # batch, L, H, P, N, G, io
    (1, 300, 2, 8, 16, 1, "f32"),
    (2, 513, 4, 64, 128, 1, "bf16"),      # three chunks, ragged
    (1, 77, 6, 5, 7, 3, "f32"),
    (2, 1, 2, 16, 32, 2, "bf16"),         # single step
    (1, 1000, 3, 40, 7, 3, "bf16"),       # two head-dim tiles, odd N, groups
    (1, 700, 2, 64, 100, 1, "bf16"),      # N not a multiple of 8
    (2, 2048, 4, 32, 64, 2, "bf16"),
    (1, 600, 2, 80, 96, 1, "bf16"),       # two 64-column head-dim slices, N tile 96
    (1, 520, 2, 20, 24, 2, "bf16"),       # P, N not multiples of 8: scalar loads
    (1, 700, 3, 64, 64, 1, "bf16"),       # odd head count per group: one head per workgroup
    (2, 1100, 6, 64, 128, 2, "bf16"),     # two heads per workgroup in each of two groups
]


def test_ssd_many_chunks_two_groups(dev):
    """Many chunks (96 per sequence) and two B / C groups: every workgroup of
    the matrix-core form reads the B and C rows of its head's group."""
    p = inputs.SSDProblem("case", 2, 24576, 8, 32, 32, 2, "bf16", 91)
    announce("ssd many chunks, two groups %s" % (p,))
    s = inputs.ssd_inputs(p)
    y, h = run_ssd(ssd_to_dev(s, p.io, dev), _lib.VARIANT_SSD_CHUNKED)
    rng = np.random.default_rng(5)
    rows = [(int(rng.integers(p.batch)), int(rng.integers(p.nheads)), int(rng.integers(p.headdim)))
            for _ in range(10)] + [(1, 7, 31), (0, 4, 0)]
    yo, ho = oracle.ssd_rows(rows, s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"], s["dt_bias"])
    ys = np.stack([y[b, :, hh, pp] for b, hh, pp in rows])
    hs = np.stack([h[b, hh, pp] for b, hh, pp in rows])
    gates.check(ys, yo, p.io, "y")
    gates.check_state(hs, ho, p.io, "h_last")


@pytest.mark.parametrize("variant", SSD_VARIANTS)
@pytest.mark.parametrize("case", SSD_SMALL)
def test_ssd_small_full_compare(dev, variant, case):
    batch, L, H, P, N, G, io = case
    if variant == _lib.VARIANT_SSD_CHUNKED and io != "bf16":
        pytest.skip("the matrix-core form takes bf16 activations only")
    announce("ssd variant=%d %s" % (variant, case))
    p = inputs.SSDProblem("case", batch, L, H, P, N, G, io, 50 + L)
    s = inputs.ssd_inputs(p)
    y, h = run_ssd(ssd_to_dev(s, io, dev), variant)
    yo, ho = oracle.ssd(s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"], s["dt_bias"])
    gates.check(ssd_rows_of(y), ssd_rows_of(yo), io, "y")
    gates.check_state(h, ho, io, "h_last")


@pytest.mark.parametrize("variant", [_lib.VARIANT_AUTO] + SSD_VARIANTS)
def test_ssd_full_size_sampled_rows(dev, variant):
    p = inputs.SSD_LAYER
    announce("ssd variant=%d workload=%s" % (variant, p.name))
    s = inputs.ssd_inputs(p)
    y, h = run_ssd(ssd_to_dev(s, p.io, dev), variant)
    rng = np.random.default_rng(3)
    rows = [(0, 0, 0), (p.batch - 1, p.nheads - 1, p.headdim - 1)] + [
        (int(rng.integers(p.batch)), int(rng.integers(p.nheads)), int(rng.integers(p.headdim)))
        for _ in range(6)]
    yo, ho = oracle.ssd_rows(rows, s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"], s["dt_bias"])
    ys = np.stack([y[b, :, hh, pp] for b, hh, pp in rows])
    hs = np.stack([h[b, hh, pp] for b, hh, pp in rows])
    gates.check(ys, yo, p.io, "y")
    gates.check_state(hs, ho, p.io, "h_last")
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_ssd_chunk_lengths_agree(dev, chunk):
    """The chunk length changes only the association order, not the result."""
    p = inputs.SSDProblem("case", 1, 1000, 2, 64, 128, 1, "bf16", 77)
    announce("ssd chunked chunk=%d" % chunk)
    s = inputs.ssd_inputs(p)
    y, h = run_ssd(ssd_to_dev(s, "bf16", dev), _lib.VARIANT_SSD_CHUNKED, chunk=chunk)
    yo, ho = oracle.ssd(s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"], s["dt_bias"])
    gates.check(ssd_rows_of(y), ssd_rows_of(yo), "bf16", "y")
    gates.check_state(h, ho, "bf16", "h_last")


def test_ssd_chunked_rejects_f32(dev):
    import selective_state_space_05_amd as mssm
    from selective_state_space_05_amd.api import MssmError, forced_variant
    p = inputs.SSDProblem("case", 1, 64, 2, 8, 16, 1, "f32", 3)
    t = ssd_to_dev(inputs.ssd_inputs(p), "f32", dev)
    with forced_variant(_lib.VARIANT_SSD_CHUNKED):
        with pytest.raises(MssmError):
            mssm.ssd_scalar_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["dt_bias"])


def test_ssd_zero_length_zero_fills_state(dev):
    import selective_state_space_05_amd as mssm
    announce("ssd L=0")
    x = torch.empty((1, 0, 2, 4), device=dev)
    dt = torch.empty((1, 0, 2), device=dev)
    B = torch.empty((1, 0, 1, 8), device=dev)
    A = -torch.ones(2, device=dev)
    h_out = torch.full((1, 2, 4, 8), 3.0, device=dev)
    y, h = mssm.ssd_scalar_fwd(x, dt, A, B, B.clone(), h_out=h_out)
    torch.cuda.synchronize()
    assert torch.all(h == 0)


def test_wrong_shaped_outputs_rejected(dev):
    """Caller-supplied out / h_out buffers of the wrong shape are refused by
    the binding before anything is queued (the C ABI sees only addresses)."""
    import selective_state_space_05_amd as mssm
    announce("wrong-shaped outputs")
    p = scan_problem(2, 64, 8, 4, "f32", 11)
    t = scan_to_dev(inputs.scan_inputs(p), "f32", dev)
    small_y = torch.full((2, 8, 32), 5.0, device=dev)
    small_h = torch.full((2, 8, 3), 5.0, device=dev)
    args = (t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"])
    with pytest.raises(ValueError):
        mssm.selective_scan_fwd(*args, out=small_y)
    with pytest.raises(ValueError):
        mssm.selective_scan_fwd(*args, h_out=small_h)
    conv_w = torch.zeros((8, 4), device=dev)
    with pytest.raises(ValueError):
        mssm.selective_scan_conv_fwd(t["u"], conv_w, t["delta"], t["A"], t["B"], t["C"],
                                     out=small_y)
    with pytest.raises(ValueError):
        mssm.selective_scan_conv_fwd(t["u"], conv_w, t["delta"], t["A"], t["B"], t["C"],
                                     h_out=small_h)
    sp = inputs.SSDProblem("case", 1, 40, 2, 8, 16, 1, "f32", 12)
    s = ssd_to_dev(inputs.ssd_inputs(sp), "f32", dev)
    sargs = (s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"], s["dt_bias"])
    with pytest.raises(ValueError):
        mssm.ssd_scalar_fwd(*sargs, out=torch.empty((1, 40, 2, 4), device=dev))
    with pytest.raises(ValueError):
        mssm.ssd_scalar_fwd(*sargs, h_out=torch.empty((1, 2, 8, 8), device=dev))
    state = torch.zeros((2, 8, 4), device=dev)
    with pytest.raises(ValueError):
        mssm.selective_state_update(state, t["u"][..., 0].contiguous(),
                                    t["delta"][..., 0].contiguous(), t["A"],
                                    t["B"][..., 0].contiguous(), t["C"][..., 0].contiguous(),
                                    out=torch.empty((2, 4), device=dev))
    torch.cuda.synchronize()
    assert torch.all(small_y == 5.0) and torch.all(small_h == 5.0)
    assert torch.all(state == 0.0)


def test_device_status_clear_after_lookback(dev):
    """A look-back run that completes leaves the device's timeout bit clear."""
    from selective_state_space_05_amd.api import device_status
    announce("device status after a look-back run")
    device_status(clear=True)
    p = scan_problem(1, 8192, 32, 16, "bf16", 8)
    run_scan(scan_to_dev(inputs.scan_inputs(p), "bf16", dev), _lib.VARIANT_LOOKBACK)
    assert device_status() & _lib.DEVICE_LOOKBACK_TIMEOUT == 0
