"""Plain float64 forward of one Mamba block with given weights (TEST
INFRASTRUCTURE ONLY).

The block as the pages describe it (reading guide glossary "Mamba Block":
input projection, 1-D convolution, selective SSM, multiplicative gate;
"Mamba / MambaMini" Q&A: a linear layer expands d_model to d_inner =
expand * d_model and splits into the SSM branch x and the gate branch z; the
Conv then an activation; a linear layer produces B, C and a low-rank Delta
that a second linear layer expands back to d_inner):

    x = x_in W_in_x,  z = x_in W_in_z                 [B, L, d_inner]
    u = SiLU(causal_conv1d(x) + conv_bias)
    dt_low = u W_x_dt, Bm = u W_x_B, Cm = u W_x_C      rank r, N, N
    dt = dt_low W_dt                                   [B, L, d_inner]
    y = scan(u, dt, A, Bm, Cm, D, z, dt_bias)          gated by SiLU(z)
    out = y W_out                                      [B, L, d_model]

Normalisation and the residual connection sit outside the block.  Matrix
products are numpy's (a library primitive); the convolution and the scan
are this package's pinned functions.
"""

import numpy as np

from .conv1d import causal_conv1d
from .scan import _f64, scan_fwd


def mamba_block_fwd(x_in, w):
    """x_in [B, L, d_model]; ``w`` a dict of weights: in_x, in_z [d_model,
    d_inner]; conv_w [d_inner, K], conv_b [d_inner]; x_dt [d_inner, r],
    x_B, x_C [d_inner, N]; dt [r, d_inner]; dt_bias, D [d_inner];
    A [d_inner, N]; out [d_inner, d_model].  Returns out [B, L, d_model]."""
    x_in = _f64(x_in)
    g = {k: _f64(v) for k, v in w.items()}
    x = x_in @ g["in_x"]
    z = x_in @ g["in_z"]
    u, _ = causal_conv1d(x, g["conv_w"], g["conv_b"])
    dt_low = u @ g["x_dt"]
    Bm = u @ g["x_B"]
    Cm = u @ g["x_C"]
    dt = dt_low @ g["dt"]
    y, _ = scan_fwd(u, dt, g["A"], Bm, Cm, g["D"], z, g["dt_bias"])
    return y @ g["out"]
