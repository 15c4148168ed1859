"""Plain float64 gradients of the selective scan (TEST INFRASTRUCTURE ONLY).

The pages name the backward pass only through its memory plan: intermediate
states are recomputed on chip during back-propagation instead of being kept
in HBM (reading guide, Hardware-aware state expansion; the aigcdaily article
"Mamba：我们所知的ChatGPT时代的终结者？", Mamba block).  What it computes is
the derivative of the forward of ``scan.py``, so this oracle is that
derivative written out by the chain rule through the recurrence: one forward
pass that keeps every state (the oracle may store what the GPU recomputes),
then one reverse-time pass with the adjoint state

    lambda_t = dL/dh_t = dy_t * C_t + Abar_{t+1} * lambda_{t+1},
    lambda_{L-1} = dy_{L-1} * C_{L-1} + dlast,

which is the same linear recurrence as the forward run backwards in time,
with decays Abar_{t+1} and inputs dy_t C_t.

Shapes as in ``scan.py``; ``dout`` [batch, L, dim] is the gradient of the
output and ``dlast`` [batch, dim, dstate] (optional) that of the final state.
Both input discretisations are differentiated.  With the exact zero-order
hold (bbar="zoh") the input coefficient is coef = (exp(Delta A) - 1)/A (Delta
where A = 0), whose derivatives are d coef/d Delta = exp(Delta A) = Abar and
d coef/d A = (Delta Abar - coef)/A, which tends to Delta^2/2 as A -> 0.
"""

import numpy as np

from .scan import _f64, softplus, silu


def _sigmoid(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def _zoh_coef_and_dA(dl, A):
    """coef = expm1(Delta A)/A and d coef/d A = Delta^2 psi(Delta A), with
    psi(x) = (x e^x - (e^x - 1))/x^2 = sum_k (k+1) x^k/(k+2)!: the closed form
    where |Delta A| >= 1e-3, the series (to x^4, truncation below 1e-15
    relative) below, where the closed form cancels."""
    x = dl[..., None] * A
    small = np.abs(x) < 1e-3
    with np.errstate(divide="ignore", invalid="ignore"):
        coef = np.where(A == 0.0, dl[..., None] * np.ones_like(A), np.expm1(x) / A)
        psi_closed = (x * np.exp(x) - np.expm1(x)) / (x * x)
    psi_series = 0.5 + x / 3.0 + x * x / 8.0 + x ** 3 / 30.0 + x ** 4 / 144.0
    psi = np.where(small, psi_series, psi_closed)
    return coef, (dl ** 2)[..., None] * psi


def scan_bwd(u, delta, A, B, C, D=None, z=None, dt_bias=None, delta_softplus=True,
             h0=None, dout=None, dlast=None, bbar="delta"):
    """Gradients of sum(dout * out) + sum(dlast * last_state).

    Returns a dict with du, ddelta (gradient of the raw dt), dA, dB, dC and,
    for the inputs that were given, dD, dz, ddt_bias, dh0.  ``bbar`` is the
    forward's input discretisation ("delta" or "zoh").
    """
    if bbar not in ("delta", "zoh"):
        raise ValueError(bbar)
    zoh = bbar == "zoh"
    u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
    D, z, dt_bias, h0 = map(_f64, (D, z, dt_bias, h0))
    dout, dlast = _f64(dout), _f64(dlast)
    bsz, L, dim = u.shape
    n = A.shape[1]

    # forward, keeping every state: H[t] = h_t, Hp[t] = h_{t-1}
    s = delta if dt_bias is None else delta + dt_bias
    dl = softplus(s) if delta_softplus else s                 # Delta [b, L, d]
    h = np.zeros((bsz, dim, n)) if h0 is None else h0.copy()
    H = np.empty((bsz, L, dim, n))
    Hp = np.empty((bsz, L, dim, n))
    Abar = np.empty((bsz, L, dim, n))
    Coef = np.empty((bsz, L, dim, n)) if zoh else None      # ZOH input coefficient
    dCoefA = np.empty((bsz, L, dim, n)) if zoh else None    # its derivative in A
    y = np.empty((bsz, L, dim))
    for t in range(L):
        Hp[:, t] = h
        Abar[:, t] = np.exp(dl[:, t, :, None] * A)
        if zoh:
            Coef[:, t], dCoefA[:, t] = _zoh_coef_and_dA(dl[:, t], A)
            h = Abar[:, t] * h + Coef[:, t] * (u[:, t, :, None] * B[:, t, None, :])
        else:
            h = Abar[:, t] * h + (dl[:, t] * u[:, t])[:, :, None] * B[:, t, None, :]
        H[:, t] = h
        y[:, t] = np.sum(h * C[:, t, None, :], axis=-1)
    if D is not None:
        y = y + D * u

    # gate: out = y * SiLU(z); d SiLU/dz = sigma(z) (1 + z (1 - sigma(z)))
    if z is not None:
        sg = _sigmoid(z)
        dy = dout * silu(z)
        dz = dout * y * sg * (1.0 + z * (1.0 - sg))
    else:
        dy = dout.copy()
        dz = None

    du = np.empty((bsz, L, dim))
    dDelta = np.empty((bsz, L, dim))
    dB = np.empty((bsz, L, n))
    dC = np.empty((bsz, L, n))
    dA = np.zeros((dim, n))
    lam_next = np.zeros((bsz, dim, n)) if dlast is None else dlast.copy()  # Abar_{t+1} lambda_{t+1}
    for t in range(L - 1, -1, -1):
        lam = dy[:, t, :, None] * C[:, t, None, :] + lam_next          # lambda_t
        dC[:, t] = np.sum(dy[:, t, :, None] * H[:, t], axis=1)         # y_t = C_t . h_t
        q = Abar[:, t] * Hp[:, t]                                      # Abar_t h_{t-1}
        if zoh:
            # h_t = Abar_t h_{t-1} + coef_t u_t B_t
            uB = u[:, t, :, None] * B[:, t, None, :]
            dB[:, t] = np.sum(lam * Coef[:, t] * u[:, t, :, None], axis=1)
            du[:, t] = np.sum(lam * Coef[:, t] * B[:, t, None, :], axis=-1)
            # d Abar/d Delta = A Abar, d coef/d Delta = Abar
            dDelta[:, t] = np.sum(lam * Abar[:, t] * (A * Hp[:, t] + uB), axis=-1)
            dA += np.sum(lam * (q * dl[:, t, :, None] + uB * dCoefA[:, t]), axis=0)
        else:
            dB[:, t] = np.sum(lam * (dl[:, t] * u[:, t])[:, :, None], axis=1)
            s1 = np.sum(lam * B[:, t, None, :], axis=-1)               # sum_n lambda B
            du[:, t] = dl[:, t] * s1
            # h_t depends on Delta through Abar_t = exp(Delta A) and Delta u B
            dDelta[:, t] = u[:, t] * s1 + np.sum(lam * q * A, axis=-1)
            dA += np.sum(lam * q * dl[:, t, :, None], axis=0)
        lam_next = Abar[:, t] * lam
    if D is not None:
        du = du + D * dy
    ds = dDelta * _sigmoid(s) if delta_softplus else dDelta          # softplus' = sigma
    res = dict(du=du, ddelta=ds, dA=dA, dB=dB, dC=dC)
    if D is not None:
        res["dD"] = np.sum(dy * u, axis=(0, 1))
    if z is not None:
        res["dz"] = dz
    if dt_bias is not None:
        res["ddt_bias"] = np.sum(ds, axis=(0, 1))
    if h0 is not None:
        res["dh0"] = lam_next                                          # Abar_0 lambda_0
    return res
