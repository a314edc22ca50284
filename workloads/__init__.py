"""Seeded synthetic inputs for the Mamba-2 SSD forward layer.

This module draws random tensors with the shapes and value distributions of
Mamba-2-shaped layers. It holds none of the SSD method's arithmetic: no
cumulative sum, no decay, no recurrence. Both sides of the parity check (the
CPU oracle under ``oracle/`` and the HIP path) consume what it returns; neither
side imports the other.

Input conventions follow the CUDA Tile Mamba-2 blog post (NVIDIA developer
blog, "Accelerating Mamba-2 with high-performance forward-pass kernels in
NVIDIA CUDA Tile"), section "Mamba-2 architecture": ``dt`` is one non-negative
scalar per (token, head), already passed through softplus; every entry of
``A`` is negative; ``x`` has ``headdim`` entries per head, ``B`` and ``C``
have ``dstate`` entries per group. Layouts are the kernel-1/2/3 listings'
index orders: x ``[batch, seqlen, nheads, headdim]``, dt ``[batch, seqlen,
nheads]``, B and C ``[batch, seqlen, ngroups, dstate]``, A and D ``[nheads]``,
states ``[batch, nheads, headdim, dstate]``.

The "N(mu, s)" in a recipe names a normal distribution with standard
deviation ``s``.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["LayerConfig", "CONFIGS", "HELD_OUT", "DECODE_CONFIGS", "config_by_name", "generate",
           "round_to_bf16", "bf16_bits_to_f32", "S6Config", "S6_CONFIGS", "s6_config_by_name", "generate_s6"]


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """One synthetic SSD layer: shapes, io dtype and value distributions."""
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    io: str                      # "f32" or "bf16": dtype of x, B, C and y
    seed: int
    dt_mu: float = -3.0          # dt = softplus(dt_sigma * z + dt_mu), z ~ N(0, 1)
    dt_sigma: float = 1.0
    dt_zero_frac: float = 0.0    # fraction of dt entries set to exactly 0
    log_negA_lo: float = 0.0     # A = -exp(U(lo, hi)) per head
    log_negA_hi: float = float(np.log(16.0))
    init_sigma: Optional[float] = None   # initial state ~ N(0, init_sigma), None = zeros
    description: str = ""

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    @property
    def nchunks(self) -> int:
        return -(-self.seqlen // self.chunk)

    def with_shape(self, **kw) -> "LayerConfig":
        """Same distributions, other sizes (for small parity variants)."""
        return dataclasses.replace(self, **kw)


CONFIGS = [
    LayerConfig("tiny", batch=1, seqlen=256, nheads=4, headdim=64, dstate=64,
                ngroups=1, chunk=64, io="f32", seed=0,
                description="tiny SSD layer, all fp32"),
    LayerConfig("mamba2-130m", batch=8, seqlen=2048, nheads=24, headdim=64,
                dstate=128, ngroups=1, chunk=256, io="bf16", seed=1,
                description="Mamba-2 130M-like layer"),
    LayerConfig("mamba2-2.7b", batch=4, seqlen=8192, nheads=80, headdim=64,
                dstate=128, ngroups=1, chunk=256, io="bf16", seed=2,
                description="Mamba-2 2.7B-like layer (headline throughput shape)"),
    LayerConfig("long-prefill", batch=1, seqlen=65536, nheads=80, headdim=64,
                dstate=128, ngroups=1, chunk=256, io="bf16", seed=3,
                init_sigma=0.1,
                description="long prefill with a nonzero initial state"),
    LayerConfig("grouped-wide", batch=2, seqlen=16384, nheads=64, headdim=128,
                dstate=256, ngroups=8, chunk=128, io="bf16", seed=4,
                dt_mu=-2.0, dt_sigma=2.0, dt_zero_frac=0.05,
                log_negA_lo=float(np.log(0.5)), log_negA_hi=float(np.log(64.0)),
                description="grouped wide-state stress: 8 heads share each B/C group"),
]

# The TileGym example shape of the CUDA Tile blog post's benchmark section
# (batch 4, 16384 tokens, 8 heads, headdim 64, dstate 128, 1 group, chunk 128),
# kept as a held-out shape that no tile choice is tuned on.
HELD_OUT = LayerConfig("tilegym-example", batch=4, seqlen=16384, nheads=8,
                       headdim=64, dstate=128, ngroups=1, chunk=128, io="bf16",
                       seed=5, description="held-out shape")


# Decode-step workloads: seqlen 1, a nonzero state standing in for the final
# state of an earlier prefill. The serving shape advances 256 sequences of the
# 2.7B-like layer by one token each; its state (671 MB fp32) dwarfs every
# other operand, which is the regime a batched decode step runs in.
DECODE_CONFIGS = [
    LayerConfig("mamba2-2.7b-decode", batch=256, seqlen=1, nheads=80, headdim=64,
                dstate=128, ngroups=1, chunk=256, io="bf16", seed=6, init_sigma=0.5,
                description="one decode step of 256 sequences, 2.7B-like layer"),
    LayerConfig("decode-small", batch=3, seqlen=1, nheads=6, headdim=64, dstate=64,
                ngroups=2, chunk=64, io="f32", seed=7, init_sigma=0.5,
                description="small decode step, fp32, 2 groups"),
]


def config_by_name(name: str) -> LayerConfig:
    for c in CONFIGS + [HELD_OUT] + DECODE_CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def round_to_bf16(a: np.ndarray):
    """Round float32 values to bfloat16, nearest-even.

    Returns ``(values, bits)``: the rounded values as float32 and their raw
    16-bit patterns (uint16), which is how a bf16 tensor is stored.
    Inputs are finite.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    bias = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    bits = ((u + bias) >> np.uint64(16)).astype(np.uint16)
    return bf16_bits_to_f32(bits), bits


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _softplus(z: np.ndarray) -> np.ndarray:
    # log(1 + e^z), evaluated without overflow.
    return np.logaddexp(0.0, z)


def generate(cfg: LayerConfig, seed: Optional[int] = None) -> dict:
    """Draw one layer's inputs.

    Draw order (fixed, so a seed names one input set): x, B, C, the dt
    normals, the dt zero mask (only when ``dt_zero_frac > 0``), the A
    uniforms, D, the initial state (only when ``init_sigma`` is set).

    Returns a dict of numpy arrays:
      x, B, C      float32 values (already rounded to bf16 when io == "bf16")
      x_bits, B_bits, C_bits   uint16 bf16 patterns (io == "bf16" only)
      dt           float32 [batch, seqlen, nheads], >= 0
      A, D         float32 [nheads], A < 0
      init_state   float32 [batch, nheads, headdim, dstate] or None
    """
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    bt, t, h, p, n, g = (cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim,
                         cfg.dstate, cfg.ngroups)
    out = {}
    for name, shape in (("x", (bt, t, h, p)), ("B", (bt, t, g, n)), ("C", (bt, t, g, n))):
        v = rng.standard_normal(shape, dtype=np.float32)
        if cfg.io == "bf16":
            v, bits = round_to_bf16(v)
            out[name + "_bits"] = bits
        out[name] = v
    z = rng.standard_normal((bt, t, h))
    dt = _softplus(cfg.dt_sigma * z + cfg.dt_mu).astype(np.float32)
    if cfg.dt_zero_frac > 0:
        dt[rng.random((bt, t, h)) < cfg.dt_zero_frac] = 0.0
    out["dt"] = dt
    out["A"] = (-np.exp(rng.uniform(cfg.log_negA_lo, cfg.log_negA_hi, h))).astype(np.float32)
    out["D"] = rng.standard_normal(h).astype(np.float32)
    if cfg.init_sigma is not None:
        out["init_state"] = (cfg.init_sigma * rng.standard_normal((bt, h, p, n))).astype(np.float32)
    else:
        out["init_state"] = None
    return out


# --------------------------------------------------------------------------
# The Mamba-1 selective scan (S6): shapes and value recipes of Sasha Rush's
# "Mamba: The Hard Way", Part 5 ("Mamba / S6"). Layouts as the page's tensors
# without singleton dimensions: x, delta [batch, channels, seqlen]; A
# [channels, dstate]; B, C [batch, dstate, seqlen]; h0 [batch, channels,
# dstate]. All float32.

@dataclasses.dataclass(frozen=True)
class S6Config:
    name: str
    batch: int
    seqlen: int
    channels: int
    dstate: int
    recipe: str          # "page": the page's create(); "random": signed, varied values
    seed: int
    h0_sigma: Optional[float] = None
    description: str = ""

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def with_shape(self, **kw) -> "S6Config":
        return dataclasses.replace(self, **kw)


S6_CONFIGS = [
    S6Config("s6-page", batch=8, seqlen=2048, channels=1024, dstate=4, recipe="page", seed=20,
             description="the page's benchmark call: mamba(*create(S=2048, Ba=8, D=1024, N=4))"),
    S6Config("s6-mamba1-130m", batch=8, seqlen=2048, channels=1536, dstate=16, recipe="random", seed=21,
             description="a Mamba-1 130M-like layer: d_inner 1536, d_state 16"),
    S6Config("s6-small", batch=2, seqlen=300, channels=100, dstate=4, recipe="random", seed=22, h0_sigma=0.5,
             description="small, ragged in both channels and tokens, with an initial state"),
]


def s6_config_by_name(name: str) -> S6Config:
    for c in S6_CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def generate_s6(cfg: S6Config, seed: Optional[int] = None) -> dict:
    """Draw one selective-scan input set (float32 numpy arrays).

    recipe "page" follows the page's create(): x ~ U[0, 1), A = -1, B = 0.1,
    C ~ 0.1 U[0, 1), delta ~ 0.1 U[0, 1). recipe "random": x, B, C ~ N(0, 1),
    A = -exp(U(-1, 1)), delta = softplus(N(0, 1) - 1). Draw order: x, delta,
    A, B, C, then h0 (only when h0_sigma is set).
    """
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    bt, L, D, N = cfg.batch, cfg.seqlen, cfg.channels, cfg.dstate
    f = np.float32
    if cfg.recipe == "page":
        x = rng.random((bt, D, L), dtype=f)
        delta = (0.1 * rng.random((bt, D, L))).astype(f)
        A = -np.ones((D, N), dtype=f)
        B = np.full((bt, N, L), 0.1, dtype=f)
        C = (0.1 * rng.random((bt, N, L))).astype(f)
    elif cfg.recipe == "random":
        x = rng.standard_normal((bt, D, L), dtype=f)
        delta = _softplus(rng.standard_normal((bt, D, L)) - 1.0).astype(f)
        A = (-np.exp(rng.uniform(-1.0, 1.0, (D, N)))).astype(f)
        B = rng.standard_normal((bt, N, L), dtype=f)
        C = rng.standard_normal((bt, N, L), dtype=f)
    else:
        raise ValueError(cfg.recipe)
    h0 = None if cfg.h0_sigma is None else (cfg.h0_sigma * rng.standard_normal((bt, D, N))).astype(f)
    return {"x": x, "delta": delta, "A": A, "B": B, "C": C, "h0": h0}
