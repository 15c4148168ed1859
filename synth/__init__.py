"""Seeded synthetic inputs for the selective scan, shared by the tests, the
smoke check and the benchmark.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the scan's arithmetic, so both the CPU oracle and the GPU
path can be fed from it without sharing any of the method.

Recipe (same for every workload):
  * generator: numpy PCG64, seed = 38000 + workload index;
  * per-tensor streams: SeedSequence(seed).spawn(8) in the fixed order
    u, dt_raw, dt0, B, C, z, state, A_random;
  * u, dt_raw, z, B, C ~ N(0, 1); decode state ~ N(0, 1) (float32);
  * dt_bias = log(expm1(dt0)) (the inverse of softplus), dt0 ~ U[1e-3, 1e-1]
    for the tiny workload and log-uniform on [1e-3, 1e-1] for the others,
    so softplus(dt_bias) lies in [1e-3, 1e-1];
  * A[d, n] = -(n + 1) (S4D-real) by default, or A = -exp(N(0, 1)) with
    ``a_init="random"``; D = 1;
  * values are drawn in float32 and rounded to bfloat16 (round to nearest
    even) where the workload stores bfloat16; the rounded values are what
    both sides receive (kept here as float32 arrays whose low 16 bits are 0).
"""

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    batch: int
    seqlen: int
    dim: int
    dstate: int
    dtype: str            # storage dtype of u, dt, z, B, C, out: "f32" | "bf16"
    decode: bool = False
    dt0_dist: str = "loguniform"
    notes: str = field(default="", compare=False)

    @property
    def seed(self) -> int:
        return 38000 + self.index


# The five workloads: a tiny one for exhaustive checks, layer shapes of the
# Mamba-130M and Mamba-2.8B models named on the pages (d_state 16,
# d_inner = 2 * d_model), a million-token sequence, and a decode step.
WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 64, 16, 4, "f32", dt0_dist="uniform"),
    "mamba130m": Workload("mamba130m", 1, 8, 2048, 1536, 16, "f32"),
    "mamba2p8b": Workload("mamba2p8b", 2, 4, 8192, 5120, 16, "bf16"),
    "seq1m": Workload("seq1m", 3, 1, 1 << 20, 256, 16, "f32"),
    "decode": Workload("decode", 4, 256, 1, 5120, 16, "bf16", decode=True),
}


def round_bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even); returns
    float32 values whose low 16 bits are zero.  NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    out = (rounded & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.float32("nan")
    return out


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def make(w, *, a_init="s4d", batch=None, seqlen=None, dim=None, dstate=None,
         seed=None):
    """Draw the inputs of workload ``w`` (a Workload or its name).

    Shape overrides (batch, seqlen, dim, dstate) keep the distributions and
    let tests draw smaller or ragged variants of a workload.  Returns a dict
    of float32 numpy arrays: u, delta (= dt_raw), z, B, C, A, D, dt_bias and,
    for decode workloads, state.  Activations are [batch, seqlen, dim] and
    B, C are [batch, seqlen, dstate]; decode arrays drop the seqlen axis.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    b = w.batch if batch is None else batch
    L = w.seqlen if seqlen is None else seqlen
    d = w.dim if dim is None else dim
    n = w.dstate if dstate is None else dstate
    ss = np.random.SeedSequence(w.seed if seed is None else seed)
    streams = [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(8)]
    g_u, g_dt, g_dt0, g_B, g_C, g_z, g_state, g_A = streams

    act = (b, d) if w.decode else (b, L, d)
    bc = (b, n) if w.decode else (b, L, n)
    u = _normal(g_u, act)
    dt = _normal(g_dt, act)
    Bm = _normal(g_B, bc)
    Cm = _normal(g_C, bc)
    z = _normal(g_z, act)
    lo, hi = 1e-3, 1e-1
    if w.dt0_dist == "uniform":
        dt0 = g_dt0.uniform(lo, hi, size=d)
    else:
        dt0 = np.exp(g_dt0.uniform(np.log(lo), np.log(hi), size=d))
    dt_bias = np.log(np.expm1(dt0)).astype(np.float32)
    if a_init == "s4d":
        A = -np.broadcast_to(np.arange(1, n + 1, dtype=np.float32), (d, n)).copy()
    elif a_init == "random":
        A = -np.exp(g_A.standard_normal(size=(d, n))).astype(np.float32)
    else:
        raise ValueError(a_init)
    Dv = np.ones(d, dtype=np.float32)
    if w.dtype == "bf16":
        u, dt, Bm, Cm, z = map(round_bf16, (u, dt, Bm, Cm, z))
    out = dict(u=u, delta=dt, z=z, B=Bm, C=Cm, A=A, D=Dv, dt_bias=dt_bias)
    if w.decode:
        out["state"] = _normal(g_state, (b, d, n))
    return out


def algorithmic_bytes(w, *, batch=None, seqlen=None, dim=None, dstate=None):
    """Bytes the method must move for one call on workload ``w``: every input
    read once, every output written once, the expanded state never stored.

    forward: (3 e_in + e_out) B L D + 2 e_in B L N + 4 (D N + 2 D) + 4 B D N
    decode:  8 B D N + (3 e_in + e_out) B D + 2 e_in B N + 4 (D N + 2 D)
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    b = w.batch if batch is None else batch
    L = w.seqlen if seqlen is None else seqlen
    d = w.dim if dim is None else dim
    n = w.dstate if dstate is None else dstate
    e = 2 if w.dtype == "bf16" else 4
    params = 4 * (d * n + 2 * d)
    if w.decode:
        return 8 * b * d * n + 4 * e * b * d + 2 * e * b * n + params
    return 4 * e * b * L * d + 2 * e * b * L * n + params + 4 * b * d * n


# Block shapes of the two Mamba models the pages name (d_inner = 2 d_model,
# d_state 16); dt_rank = ceil(d_model / 16) and conv width 4 are readings
# (the pages give neither value).
BLOCKS = {
    "mamba130m": dict(d_model=768, d_inner=1536, d_state=16, dt_rank=48, conv_width=4),
    "mamba2p8b": dict(d_model=2560, d_inner=5120, d_state=16, dt_rank=160, conv_width=4),
}


def make_block(d_model, d_inner, d_state, dt_rank, conv_width, *, batch, seqlen,
               dtype="f32", seed=38100):
    """Seeded random weights and input of one Mamba block.  Projection
    weights are N(0, 1/fan_in); conv weights N(0, 1/K); conv bias N(0, 0.1^2);
    dt_bias = log(expm1(dt0)) with dt0 log-uniform on [1e-3, 1e-1]; A is
    S4D-real -(n+1); D = 1; the input is N(0, 1).  Matrices and the input are
    rounded to bfloat16 (ties to even) when dtype is "bf16"; conv weights,
    biases, A and D stay float32.  Returns (x_in, weights)."""
    g = [np.random.Generator(np.random.PCG64(c)) for c in np.random.SeedSequence(seed).spawn(12)]

    def mat(rng, rows, cols):
        return (rng.standard_normal((rows, cols)) / np.sqrt(rows)).astype(np.float32)

    w = dict(
        in_x=mat(g[0], d_model, d_inner), in_z=mat(g[1], d_model, d_inner),
        conv_w=(g[2].standard_normal((d_inner, conv_width)) / np.sqrt(conv_width)).astype(
            np.float32),
        conv_b=(g[3].standard_normal(d_inner) * 0.1).astype(np.float32),
        x_dt=mat(g[4], d_inner, dt_rank), x_B=mat(g[5], d_inner, d_state),
        x_C=mat(g[6], d_inner, d_state), dt=mat(g[7], dt_rank, d_inner),
        dt_bias=np.log(np.expm1(np.exp(g[8].uniform(np.log(1e-3), np.log(1e-1),
                                                     d_inner)))).astype(np.float32),
        A=-np.broadcast_to(np.arange(1, d_state + 1, dtype=np.float32),
                           (d_inner, d_state)).copy(),
        D=np.ones(d_inner, dtype=np.float32),
        out=mat(g[9], d_inner, d_model))
    x_in = g[10].standard_normal((batch, seqlen, d_model)).astype(np.float32)
    if dtype == "bf16":
        for k in ("in_x", "in_z", "x_dt", "x_B", "x_C", "dt", "out"):
            w[k] = round_bf16(w[k])
        x_in = round_bf16(x_in)
    return x_in, w
