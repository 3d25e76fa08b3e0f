"""GPU parity of the selective-scan backward (mssm_selective_scan_bwd)
against the float64 oracle's reverse-mode derivative on identical inputs and
output gradients.  Needs an MI355X; marked ``gpu``.

Every gradient is float32 whatever the I/O dtype, so every comparison takes
the float32 gates (the inputs of bf16 problems are exact bf16 values for
both sides).  Normwise rows: du, ddelta, dz per (b, d) over L (like y);
dB, dC per (b, n) over L; dA per d over N; dh0 per (b, d) over N; dD and
the bias gradient as one row each.
"""
from __future__ import annotations

import numpy as np
import pytest

import gates
from oracle import oracle
from selective_state_space_05_amd import inputs
from test_parity_gpu import announce, scan_to_dev, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def f64(t):
    return None if t is None else t.float().cpu().numpy().astype(np.float64)


BWD_CASES = [
    # batch, L, dim, N, io, bias, gate, skip, with h0 / dh_last
    (2, 300, 37, 16, "f32", "per_channel", True, True, True),   # waves across two batches
    (2, 300, 64, 16, "bf16", "scalar", True, True, True),       # one batch per wave
    (1, 77, 9, 5, "f32", None, False, False, False),            # no optional inputs
    (2, 129, 20, 4, "bf16", "per_channel", True, True, False),
    (1, 50, 70, 32, "f32", "scalar", True, True, True),
    (1, 33, 10, 64, "f32", "scalar", False, True, True),        # N = 64 (limit)
    (3, 1, 5, 8, "f32", "scalar", True, True, True),            # single step
    (4, 40, 3, 12, "f32", "per_channel", True, True, True),     # 8-row waves over 3-4 batches
    (2, 1024, 640, 16, "bf16", "scalar", True, True, True),     # 80 eight-row waves per batch
]


@pytest.mark.parametrize("case", BWD_CASES)
def test_scan_backward(dev, case):
    import selective_state_space_05_amd as mssm
    batch, L, dim, N, io, bias, gate, skip, extra = case
    p = inputs.ScanProblem("case", batch, L, dim, N, io, bias, gate, skip, 800 + L + N)
    announce("scan backward %s" % (case,))
    x = inputs.scan_inputs(p)
    rng = np.random.default_rng(L + dim)
    dy = rng.standard_normal((batch, dim, L)).astype(np.float32)
    if io == "bf16":
        dy = inputs.bf16_round(dy)
    h0 = inputs.initial_state((batch, dim, N), 17) if extra else None
    dhl = inputs.initial_state((batch, dim, N), 19) if extra else None
    t = scan_to_dev({k: v for k, v in x.items() if k not in ("conv_w", "conv_b")}, io, dev)
    g = mssm.selective_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], to_dev(dy, io, dev),
                                D=t["D"], z=t["z"], delta_bias=t["delta_bias"],
                                h0=None if h0 is None else torch.from_numpy(h0).to(dev),
                                dh_last=None if dhl is None else torch.from_numpy(dhl).to(dev))
    torch.cuda.synchronize()
    o = oracle.selective_scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"],
                                  z=x["z"], delta_bias=x["delta_bias"], h0=h0, dh_last=dhl)
    f = "f32"
    gates.check(f64(g["du"]), o["du"], f, "du")
    gates.check(f64(g["ddelta"]), o["ddelta"], f, "ddelta")
    if gate:
        gates.check(f64(g["dz"]), o["dz"], f, "dz")
    gates.check_state(f64(g["dB"]), o["dB"], f, "dB")
    gates.check_state(f64(g["dC"]), o["dC"], f, "dC")
    gates.check_state(f64(g["dA"]), o["dA"], f, "dA")
    if skip:
        gates.check_state(f64(g["dD"])[None], o["dD"][None], f, "dD")
    if bias:
        gates.check_state(f64(g["ddelta_bias"])[None], o["ddelta_bias"][None], f, "ddelta_bias")
    if extra:
        gates.check_state(f64(g["dh0"]), o["dh0"], f, "dh0")


def test_scan_backward_zero_length(dev):
    """L = 0: the final state is the initial state, so dh0 = dh_last, and
    every summed gradient is zero."""
    import selective_state_space_05_amd as mssm
    announce("scan backward L=0")
    u = torch.empty((2, 3, 0), device=dev)
    A = -torch.ones((3, 4), device=dev)
    B = torch.empty((2, 4, 0), device=dev)
    dhl = torch.randn((2, 3, 4), device=dev)
    g = mssm.selective_scan_bwd(u, u.clone(), A, B, B.clone(), u.clone(), D=torch.ones(3, device=dev),
                                dh_last=dhl)
    torch.cuda.synchronize()
    assert torch.equal(g["dh0"], dhl)
    assert torch.all(g["dA"] == 0) and torch.all(g["dD"] == 0) and torch.all(g["ddelta_bias"] == 0)


def test_scan_backward_full_size():
    """The Mamba-2.8B layer's backward at full size, in the configuration the
    benchmark times (dy and dh_last drawn by inputs.output_grads, no h0).
    The oracle's backward runs over the whole layer; dA, dD and the bias
    gradient are compared in full, dB and dC over every (batch, n) row, and
    du, ddelta and dz over every (batch, channel) row."""
    import selective_state_space_05_amd as mssm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    p = inputs.BWD_PROBLEMS["mamba2.8b_layer_bwd_bf16"]
    announce("scan backward workload=%s" % p.name)
    x = inputs.scan_inputs(p)
    gr = inputs.output_grads(p)
    t = scan_to_dev({k: v for k, v in x.items() if k not in ("conv_w", "conv_b")}, p.io, dev)
    g = mssm.selective_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"],
                                to_dev(gr["dy"], p.io, dev), D=t["D"], z=t["z"],
                                delta_bias=t["delta_bias"],
                                dh_last=torch.from_numpy(gr["dh_last"]).to(dev))
    torch.cuda.synchronize()
    got = {k: f64(v) for k, v in g.items()}
    del g, t
    print("[gpu case] oracle backward over the whole layer", flush=True)
    o = oracle.selective_scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], gr["dy"], D=x["D"],
                                  z=x["z"], delta_bias=x["delta_bias"], dh_last=gr["dh_last"])
    f = "f32"
    gates.check_state(got["dA"], o["dA"], f, "dA")
    gates.check_state(got["dD"][None], o["dD"][None], f, "dD")
    gates.check_state(got["ddelta_bias"][None], o["ddelta_bias"][None], f, "ddelta_bias")
    gates.check_state(got["dB"], o["dB"], f, "dB")
    gates.check_state(got["dC"], o["dC"], f, "dC")
    gates.check(got["du"], o["du"], f, "du")
    gates.check(got["ddelta"], o["ddelta"], f, "ddelta")
    gates.check(got["dz"], o["dz"], f, "dz")


def _split_vs_blocks(p, dev, blk=1024):
    """Every (batch, channel) row's du, ddelta, dz and dh0 from one call on
    problem p must equal, bit for bit, those of calls on blocks of `blk`
    channels of one batch (at most 64 groups: never cut), with h0 and
    dh_last given.  dB and dC are compared to the blocks' sums with the
    float32 gates (their order of addition differs)."""
    import selective_state_space_05_amd as mssm
    x = inputs.scan_inputs(p)
    gr = inputs.output_grads(p)
    rng = np.random.default_rng(77)
    h0 = (0.5 * rng.standard_normal((p.batch, p.dim, p.dstate))).astype(np.float32)
    t = scan_to_dev({k: v for k, v in x.items() if k not in ("conv_w", "conv_b")}, p.io, dev)
    dy = to_dev(gr["dy"], p.io, dev)
    dhl = torch.from_numpy(gr["dh_last"]).to(dev)
    h0d = torch.from_numpy(h0).to(dev)
    opt = lambda v, sl: None if v is None else sl(v)
    full = mssm.selective_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dy, D=t["D"], z=t["z"],
                                   delta_bias=t["delta_bias"], h0=h0d, dh_last=dhl)
    torch.cuda.synchronize()
    sums = {k: torch.zeros_like(full[k]) for k in ("dB", "dC")}
    for b in range(p.batch):
        for d0 in range(0, p.dim, blk):
            d1 = min(p.dim, d0 + blk)
            print("[gpu case] block batch %d channels %d..%d" % (b, d0, d1), flush=True)
            sl = lambda v: v[b:b + 1, d0:d1].contiguous()
            ch = lambda v: v[d0:d1].contiguous()
            g = mssm.selective_scan_bwd(sl(t["u"]), sl(t["delta"]), ch(t["A"]),
                                        t["B"][b:b + 1].contiguous(), t["C"][b:b + 1].contiguous(), sl(dy),
                                        D=opt(t["D"], ch), z=opt(t["z"], sl),
                                        delta_bias=opt(t["delta_bias"], ch), h0=sl(h0d), dh_last=sl(dhl))
            torch.cuda.synchronize()
            for k in ("du", "ddelta", "dz", "dh0"):
                if full.get(k) is not None:
                    assert torch.equal(g[k][0], full[k][b, d0:d1]), (k, b, d0)
            sums["dB"][b] += g["dB"][0]
            sums["dC"][b] += g["dC"][0]
            del g
    for k in ("dB", "dC"):
        gates.check_state(f64(full[k]), f64(sums[k]), "f32", k)


def test_scan_backward_split_walk_is_bitwise_whole(dev):
    """On the Mamba-2.8B backward shape the grid of 640 (batch, 16-channel)
    groups has more groups than the device holds at once, and the groups of
    the partly empty last round are walked in parts, each starting from the
    carry an adjoint-only walk stored for it: every row must be bitwise what
    the uncut walk gives."""
    p = inputs.BWD_PROBLEMS["mamba2.8b_layer_bwd_bf16"]
    announce("scan backward split vs whole, workload=%s" % p.name)
    _split_vs_blocks(p, dev)


SPLIT_CASES = [
    # batch, L, dim, N, io, gate, skip: on 256 compute units (512 slots)
    (1, 512, 11392, 16, "bf16", True, True),    # 712 groups: the last 200 in two parts
    (2, 512, 4100, 7, "bf16", True, True),     # 514 groups, a ragged last group, N = 7: four parts
    (1, 516, 8240, 16, "f32", False, False),   # 515 groups, L % 8 != 0 (element loads), ragged last chunk
]


@pytest.mark.parametrize("case", SPLIT_CASES)
def test_scan_backward_split_walk_small_shapes(dev, case):
    batch, L, dim, N, io, gate, skip = case
    p = inputs.ScanProblem("case", batch, L, dim, N, io, "scalar", gate, skip, 31)
    announce("scan backward split vs whole %s" % (case,))
    _split_vs_blocks(p, dev)
