"""Seeded synthetic inputs for the selective scan.

This module only draws numbers and stores them; it holds none of the scan's
arithmetic, so both the GPU tests and the CPU oracle's callers can use it.

Recipe (every workload, every size):
  * numpy ``Generator(PCG64(seed))``; draws are taken in float64 in the fixed
    order u, delta_raw, z, B, C, D, U(bias), dout, state -- skipping the
    tensors a workload does not use;
  * u, z, B, C, D, dout, state ~ N(0, 1); delta_raw ~ 0.5 * N(0, 1);
  * delta_bias = log(expm1(U)), U ~ Uniform[1e-3, 1e-1] per channel: the
    inverse of softplus, so that softplus(bias) lands in that range -- the
    delta range set through the projection bias that the state-spaces/mamba
    README describes (section "Troubleshooting", "Initialization");
  * A[d, n] = -exp(log(n + 1)) computed in float64 and rounded once to
    float32 (which is exactly -(n + 1)), the same for every channel;
  * each float64 draw is rounded to float32 (round-to-nearest-even), and for
    bfloat16 storage once more from float32 to bfloat16 (nearest-even).
bfloat16 tensors are carried as uint16 bit patterns; ``widen`` returns the
exact float32 values they hold.  Batch rows are drawn all at once, so a
row's data never depends on how many rows are used afterwards (a row of a
smaller batch is a slice of the full batch).

The named workloads are the shapes of two Mamba layers (d_model 768 and 2560
with expansion 2, i.e. d_inner 1536 and 5120; state-spaces/mamba README,
"Usage" and "Pretrained Models") with d_state 16, plus a tiny correctness
case and a decode case.  No dataset, checkpoint or evaluation suite is used.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED_BASE = 20261203


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "fwd", "bwd" or "decode"
    batch: int
    dim: int
    dstate: int
    seqlen: int  # 1 for decode
    io: str  # "f32" or "bf16"
    has_z: bool = True
    has_D: bool = True
    has_bias: bool = True
    softplus: bool = True
    last_state: bool = False
    seed: int = SEED_BASE

    @property
    def elements(self) -> int:
        return self.batch * self.dim * self.seqlen


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fwd_f32_1x64x256", "fwd", 1, 64, 16, 256, "f32", seed=SEED_BASE + 0),
        Workload("mamba130m_fwd_bf16_8x1536x2048", "fwd", 8, 1536, 16, 2048, "bf16",
                 seed=SEED_BASE + 1),
        Workload("mamba2p8b_fwd_bf16_4x5120x4096", "fwd", 4, 5120, 16, 4096, "bf16",
                 last_state=True, seed=SEED_BASE + 2),
        Workload("mamba130m_bwd_f32_8x1536x2048", "bwd", 8, 1536, 16, 2048, "f32",
                 seed=SEED_BASE + 3),
        Workload("decode_bf16_256x5120", "decode", 256, 5120, 16, 1, "bf16",
                 seed=SEED_BASE + 4),
        Workload("mamba130m_bwd_bf16_8x1536x2048", "bwd", 8, 1536, 16, 2048, "bf16",
                 seed=SEED_BASE + 5),
        # a long prefill of one sequence: too few (row, state) lanes to fill
        # the chip, the case the time-segmented scan serves
        Workload("mamba130m_long_bf16_1x1536x16384", "bwd", 1, 1536, 16, 16384, "bf16",
                 seed=SEED_BASE + 6),
        # a short prefill of one sequence (384 wavefronts sequentially, for
        # 1024 SIMDs): the case of the segmented scan regime
        Workload("mamba130m_prefill_bf16_1x1536x2048", "bwd", 1, 1536, 16, 2048, "bf16",
                 seed=SEED_BASE + 7),
    ]
}


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def widen(x: np.ndarray) -> np.ndarray:
    """Exact float32 values of a stored array (float32, or uint16 bf16 bits)."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.asarray(x, dtype=np.float32)


def _store(x64: np.ndarray, io: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return bf16_bits(x32) if io == "bf16" else x32


def custom(kind: str, batch: int, dim: int, dstate: int, seqlen: int, io: str = "f32",
           seed: int = 1, **flags) -> Workload:
    """A workload of any shape with the same distributions (for tests)."""
    name = f"{kind}_{io}_{batch}x{dim}x{dstate}x{seqlen}_s{seed}"
    return Workload(name, kind, batch, dim, dstate, seqlen, io, seed=seed, **flags)


def make(w: Workload | str) -> dict:
    """Draw the arrays of a workload.

    Returns a dict with u, delta, B, C, A and, as the workload asks, z, D,
    delta_bias, dout (backward) and state (decode).  Shapes:
      scan:   u, delta, z, dout (batch, dim, L); B, C (batch, dstate, L)
      decode: u, delta, z (batch, dim); B, C (batch, dstate);
              state (batch, dim, dstate) float32
      A (dim, dstate), D and delta_bias (dim,) are always float32.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.Generator(np.random.PCG64(w.seed))
    decode = w.kind == "decode"
    row_shape = (w.batch, w.dim) if decode else (w.batch, w.dim, w.seqlen)
    bc_shape = (w.batch, w.dstate) if decode else (w.batch, w.dstate, w.seqlen)
    out = {}
    out["u"] = _store(rng.standard_normal(row_shape), w.io)
    out["delta"] = _store(0.5 * rng.standard_normal(row_shape), w.io)
    if w.has_z:
        out["z"] = _store(rng.standard_normal(row_shape), w.io)
    out["B"] = _store(rng.standard_normal(bc_shape), w.io)
    out["C"] = _store(rng.standard_normal(bc_shape), w.io)
    if w.has_D:
        out["D"] = rng.standard_normal(w.dim).astype(np.float32)
    if w.has_bias:
        U = rng.uniform(1e-3, 1e-1, w.dim)
        out["delta_bias"] = np.log(np.expm1(U)).astype(np.float32)
    if w.kind == "bwd":
        out["dout"] = _store(rng.standard_normal(row_shape), w.io)
    if decode:
        out["state"] = rng.standard_normal((w.batch, w.dim, w.dstate)).astype(np.float32)
    a_row = (-np.exp(np.log(np.arange(1, w.dstate + 1, dtype=np.float64)))).astype(np.float32)
    out["A"] = np.ascontiguousarray(np.broadcast_to(a_row, (w.dim, w.dstate)))
    return out


# ---------------------------------------------------------------------------
# Inputs of the causal convolution in front of the scan
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class ConvWorkload:
    """Shape of the causal depthwise convolution (x: batch x dim x seqlen)."""
    name: str
    batch: int
    dim: int
    seqlen: int  # 1 for a decode step
    width: int
    io: str
    has_bias: bool = True
    has_init: bool = False
    decode: bool = False
    seed: int = SEED_BASE

    @property
    def elements(self) -> int:
        return self.batch * self.dim * self.seqlen


CONV_WORKLOADS = {
    w.name: w
    for w in [
        ConvWorkload("mamba130m_conv_f32_8x1536x2048", 8, 1536, 2048, 4, "f32",
                     seed=SEED_BASE + 10),
        ConvWorkload("mamba130m_conv_bf16_8x1536x2048", 8, 1536, 2048, 4, "bf16",
                     seed=SEED_BASE + 11),
        ConvWorkload("conv_decode_bf16_256x5120", 256, 5120, 1, 4, "bf16", decode=True,
                     seed=SEED_BASE + 12),
    ]
}


def conv_custom(batch: int, dim: int, seqlen: int, width: int = 4, io: str = "f32",
                seed: int = 1, **flags) -> ConvWorkload:
    name = f"conv_{io}_{batch}x{dim}x{seqlen}_k{width}_s{seed}"
    return ConvWorkload(name, batch, dim, seqlen, width, io, seed=seed, **flags)


def make_conv(w: ConvWorkload | str) -> dict:
    """Draw the arrays of a convolution workload.

    Draw order: x, weight, bias, init (window), dout, state (decode).
    x, dout, init, state ~ N(0, 1); weight and bias ~ U(-1/sqrt(width),
    1/sqrt(width)), the default initialisation of a depthwise Conv1d layer
    (fan-in = width).  Shapes: x, dout (batch, dim, seqlen) -- (batch, dim)
    for a decode step; weight (dim, width); bias (dim,); init and state
    (batch, dim, width - 1) float32.  x and dout are stored in the io dtype,
    the rest in float32.
    """
    if isinstance(w, str):
        w = CONV_WORKLOADS[w]
    rng = np.random.Generator(np.random.PCG64(w.seed))
    row_shape = (w.batch, w.dim) if w.decode else (w.batch, w.dim, w.seqlen)
    bound = 1.0 / np.sqrt(w.width)
    out = {"x": _store(rng.standard_normal(row_shape), w.io)}
    out["weight"] = rng.uniform(-bound, bound, (w.dim, w.width)).astype(np.float32)
    if w.has_bias:
        out["bias"] = rng.uniform(-bound, bound, w.dim).astype(np.float32)
    if w.has_init:
        out["init"] = rng.standard_normal((w.batch, w.dim, w.width - 1)).astype(np.float32)
    if not w.decode:
        out["dout"] = _store(rng.standard_normal(row_shape), w.io)
    else:
        out["state"] = rng.standard_normal((w.batch, w.dim, w.width - 1)).astype(np.float32)
    return out


# ---------------------------------------------------------------------------
# Inputs of the Mamba-2 SSD scan (scalar A per head)
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class SsdWorkload:
    """Shape of an SSD forward: x (batch, seqlen, nheads, headdim)."""
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    ngroups: int
    dstate: int
    has_D: bool = True
    has_bias: bool = True
    has_h0: bool = False
    bwd: bool = False  # also draw dout and dlast (after every forward input)
    seed: int = SEED_BASE

    @property
    def elements(self) -> int:
        return self.batch * self.seqlen * self.nheads * self.headdim


SSD_WORKLOADS = {
    w.name: w
    for w in [
        # d_model 768 (the 130M size), expand 2 -> 1536 channels = 24 heads of 64,
        # d_state 128, one group
        SsdWorkload("mamba2_130m_ssd_bf16_8x2048x24x64_n128", 8, 2048, 24, 64, 1, 128,
                    seed=SEED_BASE + 30),
        SsdWorkload("mamba2_130m_ssd_bwd_bf16_8x2048x24x64_n128", 8, 2048, 24, 64, 1, 128,
                    bwd=True, seed=SEED_BASE + 31),
    ]
}


def ssd_custom(batch: int, seqlen: int, nheads: int, headdim: int, ngroups: int, dstate: int,
               seed: int = 1, **flags) -> SsdWorkload:
    name = f"ssd_{batch}x{seqlen}x{nheads}x{headdim}_g{ngroups}_n{dstate}_s{seed}"
    return SsdWorkload(name, batch, seqlen, nheads, headdim, ngroups, dstate, seed=seed, **flags)


def make_ssd(w: SsdWorkload | str) -> dict:
    """Draw the arrays of an SSD workload.

    Draw order: x, dt, B, C, U(A), D, U(dt_bias), h0, and for a backward
    workload dout (bf16) and dlast (float32), both N(0, 1).  x, B, C, D, h0 ~
    N(0, 1); dt (raw) ~ 0.5 N(0, 1); A_h = -(1 + 15 U), U ~ Uniform[0, 1],
    one per head (the decay range of the Mamba-1 A, -1 .. -16);
    dt_bias = log(expm1(U[1e-3, 1e-1])) as for the Mamba-1 delta.  x, dt, B,
    C are stored as bf16 bits; A, D, dt_bias, h0 as float32.
    """
    if isinstance(w, str):
        w = SSD_WORKLOADS[w]
    rng = np.random.Generator(np.random.PCG64(w.seed))
    out = {"x": _store(rng.standard_normal((w.batch, w.seqlen, w.nheads, w.headdim)), "bf16")}
    out["dt"] = _store(0.5 * rng.standard_normal((w.batch, w.seqlen, w.nheads)), "bf16")
    out["B"] = _store(rng.standard_normal((w.batch, w.seqlen, w.ngroups, w.dstate)), "bf16")
    out["C"] = _store(rng.standard_normal((w.batch, w.seqlen, w.ngroups, w.dstate)), "bf16")
    out["A"] = (-(1.0 + 15.0 * rng.uniform(0.0, 1.0, w.nheads))).astype(np.float32)
    if w.has_D:
        out["D"] = rng.standard_normal(w.nheads).astype(np.float32)
    if w.has_bias:
        U = rng.uniform(1e-3, 1e-1, w.nheads)
        out["dt_bias"] = np.log(np.expm1(U)).astype(np.float32)
    if w.has_h0:
        out["h0"] = rng.standard_normal((w.batch, w.nheads, w.headdim, w.dstate)).astype(np.float32)
    if w.bwd:
        out["dout"] = _store(rng.standard_normal((w.batch, w.seqlen, w.nheads, w.headdim)), "bf16")
        out["dlast"] = rng.standard_normal((w.batch, w.nheads, w.headdim, w.dstate)).astype(np.float32)
    return out
