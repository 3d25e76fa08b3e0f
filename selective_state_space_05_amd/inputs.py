"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the scan's arithmetic, so both the HIP path and the float64
oracle may use it without sharing any of the method.

Recipe (one ``numpy.random.default_rng(seed)`` stream per problem, float32
draws, affine maps in float32, then bf16 round-to-nearest-even for the
activations of bf16 problems):

  selective scan, draw order: u, delta_raw, delta_bias (when per channel),
  theta (A = -exp(theta)), B, C, D, z (when gated)
    u, B, C, D, z ~ N(0, 1)
    delta_raw     ~ N(-2, 0.5)
    delta_bias    = 0.5 for every channel ("scalar") or U(-4, -2) per channel
    theta         ~ U(0, ln 10)  -> A log-uniform in [-10, -1]; the
                    -exp(theta) form keeps every decay exp(delta*A) in (0, 1)
                    (www.mhpq.cn/news/984979 essay, section 3.1).
  SSD, draw order: x, dt_raw, dt_bias, theta (A_h = -exp(theta)), B, C, D,
  z (when gated)
    x, B, C, D, z ~ N(0, 1)
    dt_raw        ~ N(-2, 0.5)
    dt_bias       ~ U(-4, -2) per head
    theta         ~ U(0, ln 16)

  convolution prologue (when ``conv``): after z, conv_w ~ 0.5 N(0, 1) of
  shape (dim, 4) and conv_b ~ 0.1 N(0, 1) per channel; u is then the
  prologue's input.
  decode step (one time step on a cached state): the selective-scan recipe
  above with L = 1 (the length axis dropped), then from a second stream
  (seed + 1) the state ~ N(0, 1) of shape (batch, dim, N).
  initial states of the scans (``initial_state``): N(0, 1) float32 from
  their own stream.

The named workloads below carry the layer shapes the pages talk about (a
Mamba-130M layer, a Mamba-2.8B layer, a million-step sequence, a Mamba-2
layer); no dataset or trained weight is involved.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.
    NaN/Inf are not produced by the recipes and are not special-cased.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values already rounded by ``bf16_round``."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


CONV_WIDTH = 4   # the prologue's convolution width (the pages' d_conv)


@dataclasses.dataclass(frozen=True)
class ScanProblem:
    name: str
    batch: int
    seqlen: int
    dim: int
    dstate: int
    io: str                   # "f32" or "bf16"
    bias: Optional[str]       # "scalar" (0.5), "per_channel" (U(-4,-2)) or None
    gate: bool                # z present
    skip: bool                # D present
    seed: int
    conv: bool = False        # u is the input of a width-4 causal conv + SiLU prologue

    @property
    def elements(self) -> int:
        return self.batch * self.seqlen * self.dim * self.dstate

    @property
    def io_bytes(self) -> int:
        return 4 if self.io == "f32" else 2

    def min_traffic_bytes(self) -> int:
        """Every input read once and every output written once."""
        s = self.io_bytes
        act = (4 if self.gate else 3) * self.batch * self.dim * self.seqlen * s
        bc = 2 * self.batch * self.dstate * self.seqlen * s
        par = 4 * self.dim * self.dstate
        par += 4 * self.dim * ((1 if self.skip else 0) + (1 if self.bias else 0))
        par += 4 * self.dim * (CONV_WIDTH + 1) if self.conv else 0
        hl = 4 * self.batch * self.dim * self.dstate
        return act + bc + par + hl

    def replace(self, **kw) -> "ScanProblem":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class SSDProblem:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    io: str
    seed: int
    bias: bool = True
    skip: bool = True
    gate: bool = False        # z present (drawn after D)

    @property
    def elements(self) -> int:
        return self.batch * self.seqlen * self.nheads * self.headdim * self.dstate

    @property
    def io_bytes(self) -> int:
        return 4 if self.io == "f32" else 2

    def min_traffic_bytes(self) -> int:
        s = self.io_bytes
        x = self.batch * self.seqlen * self.nheads * self.headdim * s
        bc = 2 * self.batch * self.seqlen * self.ngroups * self.dstate * s
        dt = self.batch * self.seqlen * self.nheads * s
        par = 4 * self.nheads * (1 + (1 if self.bias else 0) + (1 if self.skip else 0))
        hl = 4 * self.batch * self.nheads * self.headdim * self.dstate
        return (3 if self.gate else 2) * x + bc + dt + par + hl

    def replace(self, **kw) -> "SSDProblem":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class StepProblem:
    """One decode step: a batch of sequences advanced by one time step."""
    name: str
    batch: int
    dim: int
    dstate: int
    io: str
    bias: Optional[str]
    gate: bool
    skip: bool
    seed: int

    @property
    def elements(self) -> int:
        return self.batch * self.dim * self.dstate

    @property
    def io_bytes(self) -> int:
        return 4 if self.io == "f32" else 2

    def min_traffic_bytes(self) -> int:
        """The state read and written once, every other operand once."""
        s = self.io_bytes
        state = 2 * 4 * self.batch * self.dim * self.dstate
        act = (4 if self.gate else 3) * self.batch * self.dim * s
        bc = 2 * self.batch * self.dstate * s
        par = 4 * self.dim * self.dstate
        par += 4 * self.dim * ((1 if self.skip else 0) + (1 if self.bias else 0))
        return state + act + bc + par

    def replace(self, **kw) -> "StepProblem":
        return dataclasses.replace(self, **kw)


# Named workloads.
TINY = ScanProblem("tiny_f32", 1, 64, 8, 4, "f32", "scalar", False, True, 0)
MAMBA_130M = ScanProblem("mamba130m_layer_f32", 2, 8192, 1536, 16, "f32",
                         "per_channel", True, True, 1)
MAMBA_2_8B = ScanProblem("mamba2.8b_layer_bf16", 2, 4096, 5120, 16, "bf16",
                         "scalar", True, True, 2)
MILLION = ScanProblem("million_step_bf16", 1, 1 << 20, 256, 16, "bf16",
                      "scalar", False, True, 3)
SSD_LAYER = SSDProblem("mamba2_ssd_layer_bf16", 2, 8192, 48, 64, 128, 1,
                       "bf16", 4)

# a decode step of the Mamba-2.8B layer for 256 sequences: 84 MB of state
DECODE_2_8B = StepProblem("mamba2.8b_decode_bf16", 256, 5120, 16, "bf16", "scalar",
                          True, True, 12)

# the Mamba-2.8B layer fed by its convolution prologue (u formed on chip)
MAMBA_2_8B_CONV = MAMBA_2_8B.replace(name="mamba2.8b_layer_conv_bf16", conv=True)

SCAN_PROBLEMS = {p.name: p for p in (TINY, MAMBA_130M, MAMBA_2_8B, MILLION, MAMBA_2_8B_CONV)}
# the backward of the Mamba-2.8B layer (output gradients drawn by
# ``output_grads``)
BWD_PROBLEMS = {"mamba2.8b_layer_bwd_bf16": MAMBA_2_8B.replace(name="mamba2.8b_layer_bwd_bf16")}
SSD_PROBLEMS = {SSD_LAYER.name: SSD_LAYER}
STEP_PROBLEMS = {DECODE_2_8B.name: DECODE_2_8B}


def scan_inputs(p: ScanProblem) -> dict:
    """Draw the inputs of a selective-scan problem.

    Returns float32 numpy arrays (bf16 problems: activations already rounded
    to bf16 values).  Keys: u, delta, delta_bias, A, B, C, D, z, conv_w,
    conv_b (absent operands are None).  Layouts: u, delta, z (batch, dim, L);
    B, C (batch, N, L); A (dim, N); delta_bias, D, conv_b (dim,); conv_w
    (dim, 4).  With ``conv``, u is the input of the convolution prologue.
    """
    rng = np.random.default_rng(p.seed)
    f32 = np.float32
    sh = (p.batch, p.dim, p.seqlen)
    u = rng.standard_normal(sh, dtype=f32)
    delta = rng.standard_normal(sh, dtype=f32)
    delta *= f32(0.5)
    delta += f32(-2.0)
    if p.bias == "per_channel":
        bias = rng.random(p.dim, dtype=f32) * f32(2.0) + f32(-4.0)
    elif p.bias == "scalar":
        bias = np.full(p.dim, 0.5, dtype=f32)
    else:
        bias = None
    theta = rng.random((p.dim, p.dstate), dtype=f32) * f32(math.log(10.0))
    A = -np.exp(theta)
    B = rng.standard_normal((p.batch, p.dstate, p.seqlen), dtype=f32)
    C = rng.standard_normal((p.batch, p.dstate, p.seqlen), dtype=f32)
    D = rng.standard_normal(p.dim, dtype=f32) if p.skip else None
    z = rng.standard_normal(sh, dtype=f32) if p.gate else None
    conv_w = conv_b = None
    if p.conv:
        conv_w = rng.standard_normal((p.dim, CONV_WIDTH), dtype=f32) * f32(0.5)
        conv_b = rng.standard_normal(p.dim, dtype=f32) * f32(0.1)
    if p.io == "bf16":
        u, delta, B, C = (bf16_round(a) for a in (u, delta, B, C))
        if z is not None:
            z = bf16_round(z)
    return dict(u=u, delta=delta, delta_bias=bias, A=A.astype(f32), B=B, C=C,
                D=D, z=z, conv_w=conv_w, conv_b=conv_b)


def ssd_inputs(p: SSDProblem) -> dict:
    """Draw the inputs of a Mamba-2 scalar-decay problem.

    Keys: x (batch, L, H, P), dt (batch, L, H), dt_bias (H,), A (H,),
    B, C (batch, L, G, N), D (H,), z (batch, L, H, P) or None.
    """
    rng = np.random.default_rng(p.seed)
    f32 = np.float32
    x = rng.standard_normal((p.batch, p.seqlen, p.nheads, p.headdim), dtype=f32)
    dt = rng.standard_normal((p.batch, p.seqlen, p.nheads), dtype=f32)
    dt *= f32(0.5)
    dt += f32(-2.0)
    bias = (rng.random(p.nheads, dtype=f32) * f32(2.0) + f32(-4.0)) if p.bias else None
    theta = rng.random(p.nheads, dtype=f32) * f32(math.log(16.0))
    A = (-np.exp(theta)).astype(f32)
    B = rng.standard_normal((p.batch, p.seqlen, p.ngroups, p.dstate), dtype=f32)
    C = rng.standard_normal((p.batch, p.seqlen, p.ngroups, p.dstate), dtype=f32)
    D = rng.standard_normal(p.nheads, dtype=f32) if p.skip else None
    z = rng.standard_normal(x.shape, dtype=f32) if p.gate else None
    if p.io == "bf16":
        x, dt, B, C = (bf16_round(a) for a in (x, dt, B, C))
        if z is not None:
            z = bf16_round(z)
    return dict(x=x, dt=dt, dt_bias=bias, A=A, B=B, C=C, D=D, z=z)


def initial_state(shape, seed: int) -> np.ndarray:
    """A float32 N(0, 1) initial state of the given shape."""
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)


def step_inputs(p: StepProblem) -> dict:
    """Draw the inputs of one decode step.

    Keys: x, dt, z (batch, dim); B, C (batch, N); A (dim, N); dt_bias, D
    (dim,); state (batch, dim, N) float32.  x, dt, B, C, z, A, D, dt_bias are
    the selective-scan draws of the same problem with L = 1.
    """
    q = ScanProblem(p.name, p.batch, 1, p.dim, p.dstate, p.io, p.bias, p.gate, p.skip, p.seed)
    d = scan_inputs(q)
    sq = {k: (None if d[k] is None else np.ascontiguousarray(d[k][..., 0]))
          for k in ("u", "delta", "B", "C", "z")}
    return dict(x=sq["u"], dt=sq["delta"], dt_bias=d["delta_bias"], A=d["A"], B=sq["B"],
                C=sq["C"], D=d["D"], z=sq["z"],
                state=initial_state((p.batch, p.dim, p.dstate), p.seed + 1))


def output_grads(p: ScanProblem) -> dict:
    """Gradients of a loss with respect to the scan's outputs, for its
    backward: dy ~ N(0, 1) like u (bf16-rounded for bf16 problems) and
    dh_last ~ N(0, 1) (batch, dim, N), from the stream seed + 2."""
    rng = np.random.default_rng(p.seed + 2)
    dy = rng.standard_normal((p.batch, p.dim, p.seqlen), dtype=np.float32)
    if p.io == "bf16":
        dy = bf16_round(dy)
    dhl = rng.standard_normal((p.batch, p.dim, p.dstate), dtype=np.float32)
    return dict(dy=dy, dh_last=dhl)
