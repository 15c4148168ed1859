"""Plain float64 causal depthwise conv1d + SiLU (TEST INFRASTRUCTURE ONLY).

Before the selective SSM, a Mamba block mixes each channel's recent inputs
with a short 1-D convolution and an activation ("Mamba / MambaMini" Q&A on
the Conv before the SSM: fuse local context, then a nonlinearity; reading
guide glossary "Mamba Block": input projection, 1-D convolution, selective
SSM, multiplicative gate).  The pages give neither the width nor the form;
the readings used here (one filter of width K per channel, causal so that
decoding stays constant-time, SiLU as the activation, optional bias) are
listed in the design notes.

    out[b, t, d] = act( sum_{k<K} w[d, k] * x[b, t - (K-1) + k, d] + bias[d] )

with x at negative times taken from ``init_state`` ([batch, dim, K-1], the
K-1 inputs before t = 0, oldest first) or zero.  The final state is the last
K-1 inputs, in the same layout, so a sequence can be processed in pieces and
a decode step continues it.
"""

import numpy as np

from .scan import _f64, silu


def _history(x, init_state, k):
    """[batch, K-1 + L, dim]: the K-1 earlier inputs followed by x."""
    bsz, L, dim = x.shape
    if k == 1:
        return x
    if init_state is None:
        head = np.zeros((bsz, k - 1, dim))
    else:
        head = np.transpose(init_state, (0, 2, 1))
    return np.concatenate([head, x], axis=1)


def causal_conv1d(x, w, bias=None, init_state=None, activation="silu"):
    """Returns (out [batch, L, dim], final_state [batch, dim, K-1])."""
    x, w, bias, init_state = map(_f64, (x, w, bias, init_state))
    bsz, L, dim = x.shape
    k = w.shape[1]
    xh = _history(x, init_state, k)
    acc = np.zeros((bsz, L, dim))
    for j in range(k):
        acc = acc + w[:, j] * xh[:, j:j + L]
    if bias is not None:
        acc = acc + bias
    out = silu(acc) if activation == "silu" else acc
    final = np.transpose(xh[:, xh.shape[1] - (k - 1):], (0, 2, 1))
    return out, final


def conv1d_update(state, x, w, bias=None, activation="silu"):
    """One decode step: state [batch, dim, K-1] (oldest first), x [batch, dim].
    Returns (out [batch, dim], new_state)."""
    state, x, w, bias = map(_f64, (state, x, w, bias))
    k = w.shape[1]
    window = np.concatenate([state, x[:, :, None]], axis=2)      # [b, d, K]
    acc = np.sum(window * w[None], axis=2)
    if bias is not None:
        acc = acc + bias
    out = silu(acc) if activation == "silu" else acc
    return out, window[:, :, 1:]
