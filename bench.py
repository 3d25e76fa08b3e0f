#!/usr/bin/env python3
"""Benchmark of the selective-scan forward on one MI355X.

One step = one call of the hot path (softplus step size, discretisation,
scan, output with skip term and gate, final state) over one batch of the
workload's synthetic inputs, which are already resident in HBM.  Default
workload: the Mamba-2.8B-shaped layer (batch 2, L 4096, 5120 channels,
N 16, bf16 activations, fp32 state).

Prints one JSON line:
  metric/value/unit   scan elements per second (batch * L * channels * N)
  hbm                 minimum-traffic bytes per step / kernel time, and its
                      fraction of the 8 TB/s HBM peak
  roofline            the bound of the dominant kernel (VALU issue slots,
                      see the design doc for the per-element slot count and peak)
  cpu_baseline        the float64 CPU oracle timed on this host
  parity              sampled-row comparison with the oracle

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--variant auto|rowserial|chunked|...] [--no-cpu]
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

HBM_PEAK_GBS = 8000.0
# VALU issue rate of one MI355X: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
# (non-packed fp32 lane-operations per second).
VALU_PEAK_TSLOTS = 256 * 4 * 16 * 2.4e9 / 1e12

VARIANTS = {"auto": 0, "rowserial": 1, "chunked": 2, "lookback": 3,
            "ssd_recurrent": 4, "ssd_chunked": 5}
VARIANT_NAMES = {v: k for k, v in VARIANTS.items()}


def scan_slots(p) -> float:
    """Algorithmic VALU issue slots of one selective-scan step.

    Per element (b, t, d, n): dl*A (1), 2^x (1 transcendental = 2 slots, it
    issues at half rate), (dl*u)*B (1), state FMA (1), output FMA (1) = 6.
    Per (b, t, d): softplus (exp + log = 4 slots + 3), dl*u (1), D*u (1),
    and with a gate silu (exp + rcp = 4 slots + 2) and the product (1).
    """
    per_elem = 6
    per_row_step = 4 + 3 + 1 + (1 if p.skip else 0) + (4 + 2 + 1 if p.gate else 0)
    rows_steps = p.batch * p.dim * p.seqlen
    return per_elem * p.elements + per_row_step * rows_steps


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_05_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mamba2.8b_layer_bf16")
    ap.add_argument("--variant", default="auto", choices=sorted(VARIANTS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input/output buffer sets cycled across steps (0: enough to exceed the 256 MB Infinity Cache)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_state_space_05_amd import api, inputs

    if args.workload not in inputs.SCAN_PROBLEMS:
        raise SystemExit("unknown workload %s; choose from %s" % (
            args.workload, sorted(inputs.SCAN_PROBLEMS)))
    p = inputs.SCAN_PROBLEMS[args.workload]
    dev = torch.device("cuda:0")
    print("[bench] workload %s: drawing inputs" % p.name, file=sys.stderr, flush=True)
    x = inputs.scan_inputs(p)

    io_t = torch.bfloat16 if p.io == "bf16" else torch.float32

    def upload():
        t = {}
        for k, v in x.items():
            if v is None:
                t[k] = None
            elif k in ("A", "D", "delta_bias"):
                t[k] = torch.from_numpy(v).to(dev)
            else:
                t[k] = torch.from_numpy(v).to(io_t).to(dev)
        t["y"] = torch.empty_like(t["u"])
        t["h"] = torch.empty((p.batch, p.dim, p.dstate), dtype=torch.float32, device=dev)
        return t

    footprint = p.min_traffic_bytes()
    rotate = args.rotate or max(1, min(4, -(-(1 << 30) // footprint)))
    sets = [upload() for _ in range(rotate)]
    torch.cuda.synchronize()

    variant = VARIANTS[args.variant]

    def step(i):
        t = sets[i % rotate]
        api.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"],
                               t["z"], t["delta_bias"], out=t["y"], h_out=t["h"])

    print("[bench] warmup %d, timed %d steps, %d buffer sets" % (args.warmup, args.steps, rotate),
          file=sys.stderr, flush=True)
    with api.forced_variant(variant):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        used = VARIANT_NAMES.get(api.last_variant(), str(api.last_variant()))
        stream = torch.cuda.current_stream(dev)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps
    sec = ms_step / 1e3

    value = p.elements / sec
    hbm_gbs = footprint / sec / 1e9
    slots = scan_slots(p)
    achieved_t = slots / sec / 1e12
    sha = kernel_source_sha()
    traffic = load_traffic(p.name, sha)

    out = {
        "metric": "scan elements/s (B*L*D*N) and achieved HBM GB/s as % of MI355X peak",
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded numpy draws; no dataset or trained weights)",
        "config": {"workload": p.name, "batch": p.batch, "seqlen": p.seqlen,
                   "dim": p.dim, "dstate": p.dstate, "io": p.io,
                   "gate": p.gate, "skip": p.skip, "variant": used,
                   "buffer_sets": rotate},
        "hbm": {"min_traffic_bytes": footprint, "achieved_gbs": hbm_gbs,
                "peak_gbs": HBM_PEAK_GBS, "frac": hbm_gbs / HBM_PEAK_GBS},
        "roofline": {"bound": "alu", "achieved": achieved_t, "peak": VALU_PEAK_TSLOTS,
                     "unit": "T VALU lane-slots/s", "frac": achieved_t / VALU_PEAK_TSLOTS,
                     "traffic": traffic, "slots_per_launch": slots,
                     "kernel_source_sha": sha},
    }

    if not args.no_parity:
        print("[bench] parity on sampled rows", file=sys.stderr, flush=True)
        from oracle import oracle
        t = sets[(args.steps - 1) % rotate]
        rng = np.random.default_rng(123)
        rows = [(0, 0), (p.batch - 1, p.dim - 1)] + [
            (int(rng.integers(p.batch)), int(rng.integers(p.dim))) for _ in range(6)]
        yo, ho = oracle.selective_scan_rows(rows, x["u"], x["delta"], x["A"], x["B"], x["C"],
                                            x["D"], x["z"], x["delta_bias"])
        yg = t["y"].float().cpu().numpy().astype(np.float64)
        hg = t["h"].cpu().numpy().astype(np.float64)
        ys = np.stack([yg[b, d] for b, d in rows])
        hs = np.stack([hg[b, d] for b, d in rows])

        def g1(a, r):
            return float(np.max(np.sqrt(np.sum((a - r) ** 2, -1)) /
                                np.maximum(np.sqrt(np.sum(r ** 2, -1)), 1e-300)))
        tol = 1e-4 if p.io == "f32" else 3e-3
        out["parity"] = {"rows": len(rows), "g1_y": g1(ys, yo), "g1_h_last": g1(hs, ho),
                         "tol": tol, "ok": bool(g1(ys, yo) <= tol and g1(hs, ho) <= tol)}

    if not args.no_cpu:
        from oracle import oracle
        threads = min(os.cpu_count() or 1, int(os.environ.get("OMP_NUM_THREADS", "16")), 16)
        # Bounded sample: whole rows, as many as ~15 s of CPU work at the
        # measured single-row rate (the oracle's rows are independent).
        print("[bench] CPU oracle baseline (%d threads)" % threads, file=sys.stderr, flush=True)
        t0 = time.time()
        oracle.selective_scan_rows([(0, 0)], x["u"], x["delta"], x["A"], x["B"], x["C"],
                                   x["D"], x["z"], x["delta_bias"], nthreads=1)
        per_row = max(time.time() - t0, 1e-4)
        rows_total = p.batch * p.dim
        n_rows = int(min(rows_total, max(threads, 15.0 * threads / per_row)))
        n_rows = max(threads, (n_rows // threads) * threads) if rows_total >= threads else rows_total
        n_rows = min(n_rows, rows_total)
        # a contiguous block of rows of batch 0 (then batch 1 ...)
        flat = np.arange(n_rows)
        bsel, dsel = flat // p.dim, flat % p.dim
        sub = {k: v for k, v in x.items()}
        t0 = time.time()
        done = 0
        for b in np.unique(bsel):
            ds = dsel[bsel == b]
            lo, hi = int(ds[0]), int(ds[-1]) + 1
            oracle.selective_scan(
                x["u"][b:b + 1, lo:hi], x["delta"][b:b + 1, lo:hi], x["A"][lo:hi],
                x["B"][b:b + 1], x["C"][b:b + 1],
                None if x["D"] is None else x["D"][lo:hi],
                None if x["z"] is None else x["z"][b:b + 1, lo:hi],
                None if x["delta_bias"] is None else x["delta_bias"][lo:hi],
                nthreads=threads)
            done += hi - lo
        cpu_s = time.time() - t0
        elems = done * p.seqlen * p.dstate
        out["cpu_baseline"] = {
            "value": elems / cpu_s, "unit": "elements/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d of %d (batch, channel) rows, full length %d, float64, %.1f s" % (
                done, rows_total, p.seqlen, cpu_s)}
        del sub

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
