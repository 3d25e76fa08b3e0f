#!/usr/bin/env python3
"""Benchmark of the selective-scan forward on one MI355X.

One step = one call of the hot path over one batch of the workload's
synthetic inputs, which are already resident in HBM:
  * selective scan (default): softplus step size, discretisation, scan,
    output with skip term and gate, final state;
  * SSD (--workload mamba2_ssd_layer_bf16): the Mamba-2 scalar-decay forward;
  * decode (--workload mamba2.8b_decode_bf16): one time step on a cached
    state (batch 256 of the Mamba-2.8B layer), in place.
Default workload: the Mamba-2.8B-shaped layer (batch 2, L 4096, 5120
channels, N 16, bf16 activations, fp32 state).

Prints one JSON line:
  metric/value/unit   scan elements per second (batch * L * channels * N;
                      SSD: batch * L * heads * headdim * N; decode:
                      batch * channels * N)
  hbm                 minimum-traffic bytes per step / kernel time, and its
                      fraction of the 8 TB/s HBM peak
  roofline            the bound of the dominant kernel: VALU issue slots for
                      the selective scan, bf16 matrix-core flops for SSD,
                      HBM bytes for the decode step
  cpu_baseline        the float64 CPU oracle timed on this host
  parity              sampled-row comparison with the oracle

Timing: an untimed ramp (steps until the per-launch time settles, at most
--ramp-s seconds), W untimed warmup steps, then K steps between two events
recorded on the library's stream: ms_per_step is their mean.  A second pass
of K steps with an event after every step gives "timing"'s per-launch
median, min and max.
After the timed steps the library's probes (include/mssm_probes.h) measure
the copy ceiling and the fma / 2^x / log2 x / 1/x issue rates; the roofline
charges each transcendental its measured cost and reports
t_roof = max(t_HBM, t_ALU at the measured rates).  amd-smi's clock and
temperature readings are recorded before and after the timed region.  The
CPU baseline times the oracle on one thread and on all the host threads the
process may use (OMP_NUM_THREADS, else every core).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--variant auto|rowserial|chunked|...] [--no-cpu]
                       [--no-probes] [--ramp-s S] [--copy-probe-mib M]
       python bench.py --workload NAME --steps K --warmup W --copy-probe-mib M
                       --counters FETCH_CSV WRITE_CSV      (summary only; the
                       two rocprofv3 runs pass --ramp-s 0 --no-probes, so that
                       every library dispatch is one of the W + K steps)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "scan elements/s (B*L*D*N) and achieved HBM GB/s as % of MI355X peak"
HBM_PEAK_GBS = 8000.0
# VALU issue rate of one MI355X: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
# (non-packed fp32 lane-operations per second).
VALU_PEAK_TSLOTS = 256 * 4 * 16 * 2.4e9 / 1e12
# Dense bf16 matrix-core peak of one MI355X (TFLOP/s).
MFMA_BF16_PEAK_TFLOPS = 2500.0

VARIANTS = {"auto": 0, "rowserial": 1, "chunked": 2, "lookback": 3,
            "ssd_recurrent": 4, "ssd_chunked": 5, "pairscan": 6, "pairscan2": 7}
VARIANT_NAMES = {v: k for k, v in VARIANTS.items()}


def scan_ops(p) -> dict:
    """Algorithmic vector-ALU operations of one selective-scan step, by kind
    (fma: any single-issue multiply, add or fused multiply-add; exp, log,
    rcp: the hardware 2^x, log2 x and 1/x).

    Per element (b, t, d, n): dl*A, (dl*u)*B, the state FMA and the output
    FMA (4 fma) and one 2^x.  Per (b, t, d): softplus (one 2^x, one log2 x,
    3 fma), dl*u (1), with a skip term D*u (1), with a gate silu (2^x, 1/x,
    2 fma) and the product (1), with the convolution prologue 4 FMAs and a
    silu (2^x, 1/x, 2 fma).
    """
    rows_steps = p.batch * p.dim * p.seqlen
    gate, conv = bool(p.gate), bool(getattr(p, "conv", False))
    return {
        "fma": 4 * p.elements + rows_steps * (3 + 1 + (1 if p.skip else 0) + (3 if gate else 0)
                                              + (6 if conv else 0)),
        "exp": p.elements + rows_steps * (1 + (1 if gate else 0) + (1 if conv else 0)),
        "log": rows_steps,
        "rcp": rows_steps * ((1 if gate else 0) + (1 if conv else 0)),
    }


# Issue cost of each transcendental in multiply-add slots when no probe ran:
# the probe measures v_exp_f32, v_log_f32 and v_rcp_f32 at about half the
# multiply-add rate.
DEFAULT_COSTS = {"exp": 2.0, "log": 2.0, "rcp": 2.0}


def alu_slots(ops: dict, costs: dict) -> float:
    """Multiply-add issue slots of an operation count at the given costs."""
    return ops["fma"] + sum(costs[k] * ops[k] for k in ("exp", "log", "rcp"))


def ssd_flops(p, chunk: int = 256) -> float:
    """Algorithmic matrix-core flops of the chunked SSD form, chunk length Q.

    Per (batch, chunk): the causal half of C B^T, Q(Q+1)/2 * N multiply-adds,
    once per group.  Per (batch, chunk, head): the causal intra-chunk product
    Q(Q+1)/2 * P, the chunk state P * Q * N and the inter-chunk output
    Q * N * P multiply-adds.  Two flops per multiply-add.
    """
    nchunks = -(-p.seqlen // chunk)
    q, n, hp = chunk, p.dstate, p.headdim
    tri = q * (q + 1) // 2
    per_group = tri * n
    per_head = tri * hp + hp * q * n + q * n * hp
    return 2.0 * p.batch * nchunks * (p.ngroups * per_group + p.nheads * per_head)


# The sources each workload family's kernels are compiled from.  A counter
# summary is tied to their hash, so a change to those kernels (and only to
# those) retires it.
KERNEL_SOURCES = {
    "scan_chunked": ("device_math.h", "scan_core.h", "scan_chunked.hip"),
    "scan_lookback": ("device_math.h", "scan_core.h", "scan_lookback.hip"),
    "scan_pairscan": ("device_math.h", "scan_core.h", "scan_pairscan.hip"),
    "scan_rowserial": ("device_math.h", "scan_rowserial.hip"),
    "ssd": ("device_math.h", "ssd_chunked.hip", "ssd_recurrent.hip"),
    "step": ("device_math.h", "state_update.hip"),
    "bwd": ("device_math.h", "scan_core.h", "scan_bwd_chunked.hip"),
}
# the scan workloads whose AUTO variant is the look-back kernel (long rows
# whose channels fill under four fifths of the SIMDs); the others take the
# chunked kernel
LOOKBACK_WORKLOADS = ("million_step_bf16", "mamba130m_layer_f32")


def workload_family(workload: str, used: str = None) -> str:
    """The kernel family of a workload: of the variant a run used (as
    api.last_variant() names it), else of its AUTO variant."""
    from selective_state_space_05_amd import inputs
    if workload in inputs.SCAN_PROBLEMS:
        if used is None:
            return "scan_lookback" if workload in LOOKBACK_WORKLOADS else "scan_chunked"
        return {"lookback": "scan_lookback", "pairscan": "scan_pairscan", "pairscan2": "scan_pairscan",
                "rowserial": "scan_rowserial"}.get(used, "scan_chunked")
    if workload in inputs.SSD_PROBLEMS:
        return "ssd"
    if workload in inputs.STEP_PROBLEMS:
        return "step"
    if workload in inputs.BWD_PROBLEMS:
        return "bwd"
    raise SystemExit("unknown workload %s" % workload)


def kernel_source_sha(family: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_05_amd", "csrc")
    for name in KERNEL_SOURCES[family]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, sha: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "counters_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("source_sha") != sha:
        return None
    return c.get("hbm_bytes_per_launch")


def summarize_counters(workload: str, fetch_csv: str, write_csv: str, probe_mib: int,
                       steps: int) -> dict:
    """HBM bytes per step from two rocprofv3 --pmc runs of this bench (one
    with FETCH_SIZE, one with WRITE_SIZE, both run with --copy-probe-mib).

    Each counter is scaled by the copy probe's known traffic (probe_mib MiB
    read and written) divided by what the same counter reads, per dispatch,
    for the copy kernel.  The library's kernels (mssm namespace) are summed
    over all their dispatches and divided by the number of steps the run
    made (warmup + timed + the per-launch pass).
    """
    import csv

    def read(path, counter):
        lib, copy = {}, {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                name, d, v = r["Kernel_Name"], r["Dispatch_Id"], float(r["Counter_Value"])
                if "mssm::" in name and "probe_" not in name:
                    key = name.replace("(anonymous namespace)::", "").split("(")[0]
                    key = key.replace("void ", "")
                    lib.setdefault(key, {}).setdefault(d, 0.0)
                    lib[key][d] += v
                elif "copyBuffer" in name:
                    copy[d] = copy.get(d, 0.0) + v
        # the probe's three copies are the largest copy dispatches (torch's
        # uploads of the small operands use the same copy kernel)
        probe = sorted(copy.values())[-3:]
        return lib, probe

    out = {"workload": workload, "source_sha": kernel_source_sha(workload_family(workload)),
           "copy_probe_mib": probe_mib, "steps": steps, "kernels": {}, "scale": {}}
    per_step = 0.0
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        lib, copy = read(path, counter)
        if not copy:
            raise SystemExit("no copy-probe dispatches in %s" % path)
        copy_kib = sum(copy) / len(copy)
        scale = probe_mib * 1024.0 / copy_kib
        out["scale"][counter] = scale
        out["copy_%s_kib" % counter] = copy_kib
        for name, ds in lib.items():
            k = out["kernels"].setdefault(name, {})
            k[counter + "_kib_per_dispatch"] = sum(ds.values()) / len(ds)
            k["dispatches"] = len(ds)
            per_step += sum(ds.values()) * 1024.0 * scale / steps
    out["hbm_bytes_per_launch"] = per_step
    return out


def alu_roofline(ops: dict, min_bytes: int, sec: float, peaks: dict) -> dict:
    """Roofline of a vector-ALU kernel from its operation counts.

    achieved: issue slots per second, a transcendental costing what the
    probes measured (the multiply-add rate over its own rate; DEFAULT_COSTS
    without probes), against the published VALU peak.  t_roof = max(t_HBM
    at the 8 TB/s peak, t_ALU at the rates the probes measured), and
    roof_frac = t_roof / the measured kernel time."""
    costs = peaks.get("costs") or DEFAULT_COSTS
    slots = alu_slots(ops, costs)
    a = slots / sec / 1e12
    t_hbm = min_bytes / (HBM_PEAK_GBS * 1e9)
    rates = peaks.get("valu_tlanes")
    if rates:
        t_alu = sum(ops[k] / (rates[k] * 1e12) for k in ("fma", "exp", "log", "rcp"))
    else:
        t_alu = slots / (VALU_PEAK_TSLOTS * 1e12)
    t_roof = max(t_alu, t_hbm)
    return {"bound": "alu" if t_alu >= t_hbm else "hbm", "achieved": a, "peak": VALU_PEAK_TSLOTS,
            "unit": "T VALU lane-slots/s", "frac": a / VALU_PEAK_TSLOTS,
            "slots_per_launch": slots, "ops_per_launch": ops, "slot_costs": costs,
            "t_alu_us": t_alu * 1e6, "t_hbm_us": t_hbm * 1e6, "t_roof_us": t_roof * 1e6,
            "roof_frac": t_roof / sec}


def measure_peaks(torch, dev, api, copy_mib=1024):
    """Ceilings measured on this device with the library's probes
    (include/mssm_probes.h): the streaming-copy rate over copy_mib MiB (read
    + write bytes per second, beyond the 256 MB Infinity Cache), and the
    issue rates of fma, 2^x, log2 x and 1/x in T lane-operations per second.
    Each probe runs twice untimed, then three timed launches on the current
    stream."""
    from selective_state_space_05_amd import _lib
    stream = torch.cuda.current_stream(dev)

    def timed(fn, reps=3):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    nbytes = copy_mib << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    t = timed(lambda: api.probe_copy(src, dst))
    copy_gbs = 2 * nbytes / t / 1e9
    del src, dst
    out = torch.empty(_lib.PROBE_VALU_THREADS, dtype=torch.float32, device=dev)
    rates = {}
    for name, op, iters in (("fma", _lib.PROBE_FMA, 4000), ("exp", _lib.PROBE_EXP2, 2000),
                            ("log", _lib.PROBE_LOG2, 2000), ("rcp", _lib.PROBE_RCP, 2000)):
        lane_ops = _lib.PROBE_VALU_THREADS * iters * _lib.PROBE_VALU_OPS_PER_ITER
        t = timed(lambda: api.probe_valu(op, iters, out))
        rates[name] = lane_ops / t / 1e12
    costs = {k: rates["fma"] / rates[k] for k in ("exp", "log", "rcp")}
    return {"copy_gbs": copy_gbs, "copy_mib": copy_mib, "valu_tlanes": rates, "costs": costs}


def amd_smi_snapshot():
    """Clock and temperature of GPU 0 as amd-smi reports them (a compact
    summary; the error text if amd-smi is missing or fails)."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "-t", "--json"],
                           capture_output=True, text=True, timeout=30)
    except (OSError, subprocess.SubprocessError) as e:
        return {"error": str(e)[:200]}
    if r.returncode != 0:
        return {"error": (r.stderr or r.stdout).strip()[-300:]}
    try:
        data = json.loads(r.stdout)
    except ValueError:
        return {"error": "unparsed output", "raw": r.stdout[:400]}
    out = {"gfx_clk_mhz": [], "temperature_c": {}}

    def value(v):
        if isinstance(v, dict):
            v = v.get("value")
        try:
            return float(v)
        except (TypeError, ValueError):
            return None

    def walk(o):
        if isinstance(o, dict):
            for k, v in o.items():
                if k == "clock" and isinstance(v, dict):
                    for ck, cv in v.items():
                        if ck.startswith("gfx") and isinstance(cv, dict):
                            x = value(cv.get("clk"))
                            if x is not None:
                                out["gfx_clk_mhz"].append(x)
                elif k == "temperature" and isinstance(v, dict):
                    for tk, tv in v.items():
                        x = value(tv)
                        if x is not None:
                            out["temperature_c"][tk] = x
                else:
                    walk(v)
        elif isinstance(o, list):
            for v in o:
                walk(v)

    walk(data)
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def g1(a, r):
    """Largest row-wise relative 2-norm error."""
    return float(np.max(np.sqrt(np.sum((a - r) ** 2, -1)) /
                        np.maximum(np.sqrt(np.sum(r ** 2, -1)), 1e-300)))


class ScanBench:
    """Mamba-1 selective scan: inputs, one step, parity rows, CPU baseline."""
    dtype = "f32"   # float32 arithmetic and state whatever the I/O dtype

    def __init__(self, p, dev, torch):
        from selective_state_space_05_amd import api, inputs
        self.p, self.dev, self.torch, self.api = p, dev, torch, api
        self.x = inputs.scan_inputs(p)
        self.io_t = torch.bfloat16 if p.io == "bf16" else torch.float32

    def upload(self):
        torch, p = self.torch, self.p
        t = {}
        for k, v in self.x.items():
            if v is None:
                t[k] = None
            elif k in ("A", "D", "delta_bias", "conv_w", "conv_b"):
                t[k] = torch.from_numpy(v).to(self.dev)
            else:
                t[k] = torch.from_numpy(v).to(self.io_t).to(self.dev)
        t["y"] = torch.empty_like(t["u"])
        t["h"] = torch.empty((p.batch, p.dim, p.dstate), dtype=torch.float32, device=self.dev)
        return t

    def step(self, t):
        if self.p.conv:
            self.api.selective_scan_conv_fwd(t["u"], t["conv_w"], t["delta"], t["A"], t["B"], t["C"],
                                             t["D"], t["z"], t["delta_bias"], conv_b=t["conv_b"],
                                             out=t["y"], h_out=t["h"])
        else:
            self.api.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"],
                                        t["z"], t["delta_bias"], out=t["y"], h_out=t["h"])

    def roofline(self, sec, peaks):
        return alu_roofline(scan_ops(self.p), self.p.min_traffic_bytes(), sec, peaks)

    def _u_rows(self):
        """The scan input the oracle sees: u itself, or with the convolution
        prologue the oracle's convolution of it."""
        from oracle import oracle
        x = self.x
        if not self.p.conv:
            return x["u"]
        if getattr(self, "_uc", None) is None:
            self._uc = oracle.conv1d_silu(x["u"], x["conv_w"], x["conv_b"])
        return self._uc

    def parity(self, t):
        from oracle import oracle
        p, x = self.p, self.x
        rng = np.random.default_rng(123)
        rows = [(0, 0), (p.batch - 1, p.dim - 1)] + [
            (int(rng.integers(p.batch)), int(rng.integers(p.dim))) for _ in range(6)]
        yo, ho = oracle.selective_scan_rows(rows, self._u_rows(), x["delta"], x["A"], x["B"], x["C"],
                                            x["D"], x["z"], x["delta_bias"])
        yg = t["y"].float().cpu().numpy().astype(np.float64)
        hg = t["h"].cpu().numpy().astype(np.float64)
        ys = np.stack([yg[b, d] for b, d in rows])
        hs = np.stack([hg[b, d] for b, d in rows])
        return len(rows), g1(ys, yo), g1(hs, ho)

    def cpu_baseline(self, threads, budget_s=8.0, min_wall_s=2.0):
        """Time the oracle on whole (batch, channel) rows: as many as about
        `budget_s` seconds of work at the measured single-row rate, in passes
        repeated for at least `min_wall_s` seconds."""
        from oracle import oracle
        p, x = self.p, self.x
        u = self._u_rows()
        t0 = time.time()
        oracle.selective_scan_rows([(0, 0)], u, x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"],
                                   x["delta_bias"], nthreads=1)
        per_row = max(time.time() - t0, 1e-4)
        rows_total = p.batch * p.dim
        n_rows = int(min(rows_total, max(threads, budget_s * threads / per_row)))
        if rows_total >= threads:
            n_rows = max(threads, (n_rows // threads) * threads)
        n_rows = min(n_rows, rows_total)
        flat = np.arange(n_rows)
        bsel, dsel = flat // p.dim, flat % p.dim
        # whole passes over the sample, repeated until at least min_wall_s
        # of wall time has gone by (a pass over a whole layer can take well
        # under a second on many cores)
        t0 = time.time()
        done = 0
        passes = 0
        while True:
            for b in np.unique(bsel):
                ds = dsel[bsel == b]
                lo, hi = int(ds[0]), int(ds[-1]) + 1
                args = (x["delta"][b:b + 1, lo:hi], x["A"][lo:hi], x["B"][b:b + 1], x["C"][b:b + 1],
                        None if x["D"] is None else x["D"][lo:hi],
                        None if x["z"] is None else x["z"][b:b + 1, lo:hi],
                        None if x["delta_bias"] is None else x["delta_bias"][lo:hi])
                if p.conv:
                    oracle.selective_scan_conv(x["u"][b:b + 1, lo:hi], x["conv_w"][lo:hi],
                                               x["conv_b"][lo:hi], *args, nthreads=threads)
                else:
                    oracle.selective_scan(x["u"][b:b + 1, lo:hi], *args, nthreads=threads)
                done += hi - lo
            passes += 1
            if time.time() - t0 >= min_wall_s:
                break
        cpu_s = time.time() - t0
        elems = done * p.seqlen * p.dstate
        return elems / cpu_s, ("%d of %d (batch, channel) rows, full length %d, float64, %d pass(es), "
                               "%.1f s wall" % (n_rows, rows_total, p.seqlen, passes, cpu_s))

    def config(self):
        p = self.p
        return {"workload": p.name, "batch": p.batch, "seqlen": p.seqlen, "dim": p.dim,
                "dstate": p.dstate, "io": p.io, "gate": p.gate, "skip": p.skip, "conv": p.conv}


class SSDBench:
    """Mamba-2 scalar-decay forward."""
    dtype = "bf16"  # bf16 matrix-core products (two-term splits), float32 accumulation

    def __init__(self, p, dev, torch, chunk=256):
        from selective_state_space_05_amd import api, inputs
        self.p, self.dev, self.torch, self.api, self.chunk = p, dev, torch, api, chunk
        self.x = inputs.ssd_inputs(p)
        self.io_t = torch.bfloat16 if p.io == "bf16" else torch.float32

    def upload(self):
        torch, p = self.torch, self.p
        t = {}
        for k, v in self.x.items():
            if v is None:
                t[k] = None
            elif k in ("A", "D", "dt_bias"):
                t[k] = torch.from_numpy(v).to(self.dev)
            else:
                t[k] = torch.from_numpy(v).to(self.io_t).to(self.dev)
        t["y"] = torch.empty_like(t["x"])
        t["h"] = torch.empty((p.batch, p.nheads, p.headdim, p.dstate), dtype=torch.float32,
                             device=self.dev)
        return t

    def step(self, t):
        self.api.ssd_scalar_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["dt_bias"],
                                chunk=self.chunk, out=t["y"], h_out=t["h"])

    def roofline(self, sec, peaks):
        fl = ssd_flops(self.p, self.chunk)
        a = fl / sec / 1e12
        t_mfma = fl / (MFMA_BF16_PEAK_TFLOPS * 1e12)
        t_hbm = self.p.min_traffic_bytes() / (HBM_PEAK_GBS * 1e9)
        t_roof = max(t_mfma, t_hbm)
        return {"bound": "mfma", "achieved": a, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": a / MFMA_BF16_PEAK_TFLOPS,
                "flops_per_launch": fl, "t_mfma_us": t_mfma * 1e6, "t_hbm_us": t_hbm * 1e6,
                "t_roof_us": t_roof * 1e6, "roof_frac": t_roof / sec}

    def parity(self, t):
        from oracle import oracle
        p, s = self.p, self.x
        rng = np.random.default_rng(3)
        rows = [(0, 0, 0), (p.batch - 1, p.nheads - 1, p.headdim - 1)] + [
            (int(rng.integers(p.batch)), int(rng.integers(p.nheads)),
             int(rng.integers(p.headdim))) for _ in range(6)]
        yo, ho = oracle.ssd_rows(rows, s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"],
                                 s["dt_bias"])
        yg = t["y"].float().cpu().numpy().astype(np.float64)
        hg = t["h"].cpu().numpy().astype(np.float64)
        ys = np.stack([yg[b, :, hh, pp] for b, hh, pp in rows])
        hs = np.stack([hg[b, hh, pp] for b, hh, pp in rows])
        return len(rows), g1(ys, yo), g1(hs, ho)

    def cpu_baseline(self, threads, budget_s=6.0):
        """Time the oracle on whole (batch, head) blocks, as many as about
        `budget_s` seconds of work at the measured single-head rate."""
        from oracle import oracle
        p, s = self.p, self.x
        G = p.ngroups
        hpg = p.nheads // G

        def run(b, h0, h1, nth):
            g0 = h0 // hpg
            g1_ = (h1 - 1) // hpg + 1
            # heads [h0, h1) that share groups [g0, g1_) with the full problem
            oracle.ssd(s["x"][b:b + 1, :, h0:h1], s["dt"][b:b + 1, :, h0:h1], s["A"][h0:h1],
                       s["B"][b:b + 1, :, g0:g1_], s["C"][b:b + 1, :, g0:g1_],
                       None if s["D"] is None else s["D"][h0:h1],
                       None if s["dt_bias"] is None else s["dt_bias"][h0:h1], nthreads=nth)

        t0 = time.time()
        run(0, 0, hpg if G > 1 else 1, 1)
        per_head = max(time.time() - t0, 1e-4) / (hpg if G > 1 else 1)
        heads_total = p.batch * p.nheads
        want = int(max(1, min(heads_total, budget_s * threads / per_head)))
        if G == 1:
            nh = min(p.nheads, want)
            t0 = time.time()
            run(0, 0, nh, threads)
            done = nh
        else:
            ng = max(1, min(G, want // hpg))
            t0 = time.time()
            run(0, 0, ng * hpg, threads)
            done = ng * hpg
        cpu_s = time.time() - t0
        elems = done * p.seqlen * p.headdim * p.dstate
        return elems / cpu_s, "%d of %d (batch, head) blocks, full length %d, float64, %.1f s" % (
            done, heads_total, p.seqlen, cpu_s)

    def config(self):
        p = self.p
        return {"workload": p.name, "batch": p.batch, "seqlen": p.seqlen, "nheads": p.nheads,
                "headdim": p.headdim, "dstate": p.dstate, "ngroups": p.ngroups, "io": p.io,
                "chunk": self.chunk}


def bwd_ops(p) -> dict:
    """Algorithmic vector-ALU operations of one backward, by kind.

    Per element (b, t, d, n): the forward recomputed twice (state pass and
    segment recompute: dl*A, (dl*u)*B, FMA and a 2^x each) and the reverse
    step (dh FMA, dC product, dA 2, dB product, du FMA, d(dl) 2, carry, and
    a 2^x): 14 fma and 3 exp.  Per (b, t, d): softplus three times (2^x,
    log2 x, 3 fma each), the logistic of x (2^x, 1/x), two products and,
    with a gate, its silu and derivative (2^x, 1/x, 6 fma).
    """
    rows_steps = p.batch * p.dim * p.seqlen
    g = 1 if p.gate else 0
    return {"fma": 14 * p.elements + rows_steps * (9 + 2 + 6 * g),
            "exp": 3 * p.elements + rows_steps * (3 + 1 + g),
            "log": 3 * rows_steps,
            "rcp": rows_steps * (1 + g)}


def bwd_min_traffic_bytes(p) -> int:
    """Every input of the backward read once and every gradient written once:
    u, delta, dy (and z) in the I/O dtype, B and C, A, D, the bias and
    dh_last; du, ddelta (and dz) float32 like u, dB and dC float32 like B,
    dA, dD, the bias gradient and dh0."""
    s = 2 if p.io == "bf16" else 4
    rows_l = p.batch * p.dim * p.seqlen
    bc_l = p.batch * p.dstate * p.seqlen
    nact = 4 if p.gate else 3
    reads = nact * rows_l * s + 2 * bc_l * s + 4 * p.dim * p.dstate
    reads += 4 * p.dim * ((1 if p.skip else 0) + (1 if p.bias else 0))
    reads += 4 * p.batch * p.dim * p.dstate                     # dh_last
    writes = (nact - 1) * rows_l * 4 + 2 * bc_l * 4 + 4 * p.dim * p.dstate
    writes += 4 * p.dim * 2 + 4 * p.batch * p.dim * p.dstate    # dD, dbias, dh0
    return reads + writes


class BwdBench(ScanBench):
    """Backward of the selective scan (mssm_selective_scan_bwd)."""

    def __init__(self, p, dev, torch):
        super().__init__(p, dev, torch)
        from selective_state_space_05_amd import inputs
        self.g = inputs.output_grads(p)

    def upload(self):
        t = super().upload()
        t["dy"] = self.torch.from_numpy(self.g["dy"]).to(self.io_t).to(self.dev)
        t["dh_last"] = self.torch.from_numpy(self.g["dh_last"]).to(self.dev)
        return t

    def step(self, t):
        t["grads"] = self.api.selective_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["dy"],
                                                 D=t["D"], z=t["z"], delta_bias=t["delta_bias"],
                                                 dh_last=t["dh_last"])

    def roofline(self, sec, peaks):
        return alu_roofline(bwd_ops(self.p), bwd_min_traffic_bytes(self.p), sec, peaks)

    def min_traffic_bytes(self):
        return bwd_min_traffic_bytes(self.p)

    def _row_oracle(self, b, d, nthreads=0):
        from oracle import oracle
        x, g = self.x, self.g
        sl = lambda a: None if a is None else a[b:b + 1, d:d + 1]   # noqa: E731
        pr = lambda a: None if a is None else a[d:d + 1]            # noqa: E731
        return oracle.selective_scan_bwd(sl(x["u"]), sl(x["delta"]), pr(x["A"]), x["B"][b:b + 1],
                                         x["C"][b:b + 1], sl(g["dy"]), D=pr(x["D"]), z=sl(x["z"]),
                                         delta_bias=pr(x["delta_bias"]),
                                         dh_last=g["dh_last"][b:b + 1, d:d + 1])

    def parity(self, t):
        """du and ddelta of sampled rows depend on their row alone: the
        oracle's backward of that row gives them exactly."""
        p = self.p
        rng = np.random.default_rng(321)
        rows = [(0, 0), (p.batch - 1, p.dim - 1)] + [
            (int(rng.integers(p.batch)), int(rng.integers(p.dim))) for _ in range(2)]
        du = t["grads"]["du"].float().cpu().numpy().astype(np.float64)
        dd = t["grads"]["ddelta"].float().cpu().numpy().astype(np.float64)
        gu, gd = [], []
        for b, d in rows:
            o = self._row_oracle(b, d)
            gu.append((du[b, d], o["du"][0, 0]))
            gd.append((dd[b, d], o["ddelta"][0, 0]))
        return (len(rows), g1(np.stack([a for a, _ in gu]), np.stack([r for _, r in gu])),
                g1(np.stack([a for a, _ in gd]), np.stack([r for _, r in gd])))

    def cpu_baseline(self, threads, budget_s=6.0):
        """The oracle's backward on whole rows for about ``budget_s``: one
        row per call (the oracle's backward is single-threaded), with
        ``threads`` calls in flight on as many Python threads (the calls
        release the interpreter lock)."""
        import concurrent.futures
        p = self.p
        t0 = time.time()
        done = 0
        with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
            while done == 0 or time.time() - t0 < budget_s:
                rows = [((done + i) % p.batch, (done + i) % p.dim) for i in range(threads)]
                list(ex.map(lambda r: self._row_oracle(*r), rows))
                done += threads
        cpu_s = time.time() - t0
        return done * p.seqlen * p.dstate / cpu_s, "%d (batch, channel) rows, full length %d, float64, %.1f s" % (
            done, p.seqlen, cpu_s)

    def config(self):
        c = super().config()
        c["pass"] = "backward"
        return c


class StepBench:
    """One decode step (selective_state_update) on a cached float32 state."""
    dtype = "f32"

    def __init__(self, p, dev, torch):
        from selective_state_space_05_amd import api, inputs
        self.p, self.dev, self.torch, self.api = p, dev, torch, api
        self.x = inputs.step_inputs(p)
        self.io_t = torch.bfloat16 if p.io == "bf16" else torch.float32

    def upload(self):
        torch = self.torch
        t = {}
        for k, v in self.x.items():
            if v is None:
                t[k] = None
            elif k in ("A", "D", "dt_bias", "state"):
                t[k] = torch.from_numpy(v).to(self.dev)
            else:
                t[k] = torch.from_numpy(v).to(self.io_t).to(self.dev)
        t["y"] = torch.empty_like(t["x"])
        return t

    def step(self, t):
        self.api.selective_state_update(t["state"], t["x"], t["dt"], t["A"], t["B"], t["C"],
                                        t["D"], t["z"], t["dt_bias"], out=t["y"])

    def roofline(self, sec, peaks):
        nbytes = self.p.min_traffic_bytes()
        a = nbytes / sec / 1e9
        t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
        return {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": a / HBM_PEAK_GBS, "bytes_per_launch": nbytes, "t_roof_us": t_hbm * 1e6,
                "roof_frac": t_hbm / sec}

    def _oracle(self, nthreads=0):
        from oracle import oracle
        x = self.x
        col = lambda a: None if a is None else a[..., None]   # noqa: E731
        return oracle.selective_scan(col(x["x"]), col(x["dt"]), x["A"], col(x["B"]),
                                     col(x["C"]), x["D"], col(x["z"]), x["dt_bias"],
                                     h0=x["state"], nthreads=nthreads)

    def parity(self, t):
        """One step from the drawn state (the timed steps advanced the
        uploaded copies), compared with the oracle over every row."""
        torch = self.torch
        fresh = dict(t)
        fresh["state"] = torch.from_numpy(self.x["state"]).to(self.dev)
        fresh["y"] = torch.empty_like(t["x"])
        self.step(fresh)
        torch.cuda.synchronize()
        yo, ho = self._oracle()
        yg = fresh["y"].float().cpu().numpy().astype(np.float64)
        hg = fresh["state"].cpu().numpy().astype(np.float64)
        return self.p.batch, g1(yg, yo[..., 0]), g1(hg, ho)

    def cpu_baseline(self, threads, budget_s=4.0):
        """The oracle on the whole step, repeated for about `budget_s`."""
        reps, t0 = 0, time.time()
        while reps == 0 or time.time() - t0 < budget_s:
            self._oracle(nthreads=threads)
            reps += 1
        cpu_s = time.time() - t0
        return reps * self.p.elements / cpu_s, "the whole step (%d rows) %d times, float64, %.1f s" % (
            self.p.batch * self.p.dim, reps, cpu_s)

    def config(self):
        p = self.p
        return {"workload": p.name, "batch": p.batch, "dim": p.dim, "dstate": p.dstate,
                "io": p.io, "gate": p.gate, "skip": p.skip}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10,
                    help="untimed steps before the timed ones (also lets the GPU clock ramp up)")
    ap.add_argument("--workload", default="mamba2.8b_layer_bf16")
    ap.add_argument("--variant", default="auto", choices=sorted(VARIANTS))
    ap.add_argument("--chunk", type=int, default=256, help="SSD chunk length")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the copy and ALU peak probes (transcendentals then cost 2 slots) "
                         "and the amd-smi clock snapshots: the profiler passes, whose preloaded "
                         "library would also attach to amd-smi's own process")
    ap.add_argument("--ramp-s", type=float, default=2.0,
                    help="at most this many seconds of untimed steps before the warmup, until the "
                         "per-launch time settles (0: none)")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input/output buffer sets cycled across steps (0: enough to exceed the "
                         "256 MB Infinity Cache)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed steps, copy a buffer of this many MiB three times "
                         "(a plain kernel of known traffic for calibrating HBM byte counters)")
    ap.add_argument("--counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: summarize the counter_collection.csv files of two "
                         "rocprofv3 --pmc runs of this bench (FETCH_SIZE, then WRITE_SIZE; "
                         "same --workload/--steps/--warmup/--copy-probe-mib) into "
                         "profiles/counters_<workload>.json")
    args = ap.parse_args()

    if args.counters:
        if args.copy_probe_mib <= 0:
            raise SystemExit("--counters needs the --copy-probe-mib the runs used")
        # the runs made W warm-up steps, K timed steps and K per-launch steps
        res = summarize_counters(args.workload, args.counters[0], args.counters[1],
                                 args.copy_probe_mib, 2 * args.steps + args.warmup)
        path = os.path.join(ROOT, "profiles", "counters_%s.json" % args.workload)
        with open(path, "w") as f:
            json.dump(res, f, indent=1)
            f.write("\n")
        print(json.dumps(res))
        return

    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_state_space_05_amd import api, inputs

    dev = torch.device("cuda:0")
    if args.workload in inputs.SCAN_PROBLEMS:
        p = inputs.SCAN_PROBLEMS[args.workload]
        print("[bench] workload %s: drawing inputs" % p.name, file=sys.stderr, flush=True)
        wb = ScanBench(p, dev, torch)
    elif args.workload in inputs.SSD_PROBLEMS:
        p = inputs.SSD_PROBLEMS[args.workload]
        print("[bench] workload %s: drawing inputs" % p.name, file=sys.stderr, flush=True)
        wb = SSDBench(p, dev, torch, args.chunk)
    elif args.workload in inputs.STEP_PROBLEMS:
        p = inputs.STEP_PROBLEMS[args.workload]
        print("[bench] workload %s: drawing inputs" % p.name, file=sys.stderr, flush=True)
        wb = StepBench(p, dev, torch)
    elif args.workload in inputs.BWD_PROBLEMS:
        p = inputs.BWD_PROBLEMS[args.workload]
        print("[bench] workload %s: drawing inputs" % p.name, file=sys.stderr, flush=True)
        wb = BwdBench(p, dev, torch)
    else:
        raise SystemExit("unknown workload %s; choose from %s" % (
            args.workload, sorted(inputs.SCAN_PROBLEMS) + sorted(inputs.SSD_PROBLEMS) +
            sorted(inputs.STEP_PROBLEMS) + sorted(inputs.BWD_PROBLEMS)))

    footprint = wb.min_traffic_bytes() if hasattr(wb, "min_traffic_bytes") else p.min_traffic_bytes()
    rotate = args.rotate or max(1, min(4, -(-(1 << 30) // footprint)))
    sets = [wb.upload() for _ in range(rotate)]
    torch.cuda.synchronize()
    smi_before = None if args.no_probes else amd_smi_snapshot()

    variant = VARIANTS[args.variant]
    # the library launches on torch's current stream; every event is
    # recorded on that same stream
    stream = torch.cuda.current_stream(dev)
    with api.forced_variant(variant):
        print("[bench] clock ramp", file=sys.stderr, flush=True)
        ramp = ramp_up(torch, stream, lambda i: wb.step(sets[i % rotate]), args.ramp_s)
        print("[bench] warmup %d, timed %d steps, %d buffer sets" % (args.warmup, args.steps, rotate),
              file=sys.stderr, flush=True)
        for i in range(args.warmup):
            wb.step(sets[i % rotate])
        torch.cuda.synchronize()
        used = VARIANT_NAMES.get(api.last_variant(), str(api.last_variant()))
        # the K timed steps between one event pair: ms_per_step
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            wb.step(sets[i % rotate])
        e1.record(stream)
        torch.cuda.synchronize()
        total_ms = e0.elapsed_time(e1)
        # then K more with an event after every step, for the per-launch
        # median / min / max (an event record per step slows the host loop,
        # which for a kernel of a few tens of us shows up as idle gaps, so
        # these are not the timed steps)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(args.steps):
            wb.step(sets[i % rotate])
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
    per_launch = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    smi_after = None if args.no_probes else amd_smi_snapshot()
    ms_step = total_ms / args.steps
    sec = ms_step / 1e3

    peaks = {}
    if not args.no_probes:
        print("[bench] peak probes", file=sys.stderr, flush=True)
        peaks = measure_peaks(torch, dev, api)

    hbm_gbs = footprint / sec / 1e9
    roof = wb.roofline(sec, peaks)
    sha = kernel_source_sha(workload_family(p.name, used if p.name in inputs.SCAN_PROBLEMS else None))
    roof["traffic"] = load_traffic(p.name, sha)
    roof["kernel_source_sha"] = sha
    cfg = wb.config()
    cfg.update({"variant": used, "buffer_sets": rotate})
    from selective_state_space_05_amd import _lib

    out = {
        "metric": METRIC,
        "value": p.elements / sec,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wb.dtype,
        "data": "synthetic (seeded numpy draws; no dataset or trained weights)",
        "config": cfg,
        "timing": {"mean_us": ms_step * 1e3, "median_us": per_launch[len(per_launch) // 2] * 1e3,
                   "min_us": per_launch[0] * 1e3, "max_us": per_launch[-1] * 1e3,
                   "per_launch_mean_us": sum(per_launch) / len(per_launch) * 1e3,
                   "launches": args.steps, "ramp": ramp},
        "hbm": {"min_traffic_bytes": footprint, "achieved_gbs": hbm_gbs,
                "peak_gbs": HBM_PEAK_GBS, "frac": hbm_gbs / HBM_PEAK_GBS},
        "roofline": roof,
        "peaks_measured": peaks or None,
        "gpu_state": {"before": smi_before, "after": smi_after},
        "lib_source_hash": _lib.lib().mssm_source_hash().decode(),
    }
    if peaks:
        out["copy_ceiling_gbs"] = peaks["copy_gbs"]
        out["hbm"]["frac_of_copy_ceiling"] = hbm_gbs / peaks["copy_gbs"]

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 18          # float32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_probe_bytes_each_way"] = n * 4
        del src, dst

    if not args.no_parity:
        print("[bench] parity on sampled rows", file=sys.stderr, flush=True)
        t = sets[(args.steps - 1) % rotate]
        nrows, ey, eh = wb.parity(t)
        tol = 1e-4 if p.io == "f32" else 3e-3
        out["parity"] = {"rows": nrows, "g1_y": ey, "g1_h_last": eh, "tol": tol,
                         "ok": bool(ey <= tol and eh <= tol)}

    if not args.no_cpu:
        # all host threads this process may use: the CPU share set by
        # OMP_NUM_THREADS where the environment sets one, else every core
        share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
        threads = max(1, min(os.cpu_count() or 1, share))
        print("[bench] CPU oracle baseline: 1 thread, then %d threads" % threads,
              file=sys.stderr, flush=True)
        v1, sample1 = wb.cpu_baseline(1)
        vn, samplen = wb.cpu_baseline(threads)
        out["cpu_baseline"] = {"value": vn, "unit": "elements/s", "cores": threads,
                               "kind": "oracle", "sample": samplen,
                               "single_thread": {"value": v1, "sample": sample1},
                               "cpu_count": os.cpu_count(), "cpu_model": cpu_model()}

    print(json.dumps(out), flush=True)


def ramp_up(torch, stream, step, max_s, min_s=0.5, batch_ms=20.0, tol=0.015):
    """Untimed steps until the per-launch time settles (the GPU clock ramps
    up under load): batches of about batch_ms, until two consecutive batch
    means agree within tol after at least min_s, or max_s has passed."""
    if max_s <= 0:
        return None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.time()
    n = 1
    means, i = [], 0
    while True:
        e0.record(stream)
        for _ in range(n):
            step(i)
            i += 1
        e1.record(stream)
        torch.cuda.synchronize()
        means.append(e0.elapsed_time(e1) / n)
        n = max(1, int(batch_ms / max(means[-1], 1e-3)))
        el = time.time() - t0
        if (el >= min_s and len(means) >= 3 and abs(means[-1] - means[-2]) <= tol * means[-1]) \
                or el >= max_s:
            break
    return {"steps": i, "seconds": round(time.time() - t0, 3), "first_us": means[0] * 1e3,
            "last_us": means[-1] * 1e3, "batches": len(means)}


if __name__ == "__main__":
    main()
