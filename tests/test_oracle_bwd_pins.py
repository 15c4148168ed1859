"""Pins of the oracle's backward (oracle.scan_bwd) against facts that do not
come from it: central finite differences of the forward oracle in float64,
and closed forms of special cases.  The pages give the backward only as
"recompute the states instead of storing them" (reading guide,
Hardware-aware state expansion); the gradient itself is fixed by calculus.
"""

import numpy as np
import pytest

import oracle


def _case(seed, b=2, L=9, d=3, n=4, gate=True, h0=True, bias=True, D=True):
    r = np.random.default_rng(seed)
    c = dict(
        u=r.standard_normal((b, L, d)),
        delta=r.standard_normal((b, L, d)),
        A=-np.exp(r.standard_normal((d, n))),
        B=r.standard_normal((b, L, n)),
        C=r.standard_normal((b, L, n)),
        D=r.standard_normal(d) if D else None,
        z=r.standard_normal((b, L, d)) if gate else None,
        dt_bias=r.uniform(-2, 0, d) if bias else None,
        h0=r.standard_normal((b, d, n)) if h0 else None,
    )
    w = dict(dout=r.standard_normal((b, L, d)), dlast=r.standard_normal((b, d, n)))
    return c, w


def _loss(c, w, softplus=True):
    out, last = oracle.scan_fwd(**c, delta_softplus=softplus)
    return float(np.sum(out * w["dout"]) + np.sum(last * w["dlast"]))


def _fd(c, w, key, softplus=True, eps=1e-6):
    x = c[key]
    g = np.empty_like(x)
    for i in np.ndindex(x.shape):
        cp = dict(c)
        xp = x.copy()
        xp[i] += eps
        cp[key] = xp
        lp = _loss(cp, w, softplus)
        xp[i] -= 2 * eps
        lm = _loss(cp, w, softplus)
        g[i] = (lp - lm) / (2 * eps)
    return g


GRADS = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
         "z": "dz", "dt_bias": "ddt_bias", "h0": "dh0"}


@pytest.mark.parametrize("softplus", [True, False])
def test_every_gradient_matches_finite_differences(softplus):
    c, w = _case(200, gate=True, h0=True)
    if not softplus:
        c["delta"] = np.abs(c["delta"]) * 0.3
        c["dt_bias"] = np.full(3, 0.05)
    g = oracle.scan_bwd(**c, delta_softplus=softplus, **w)
    for key, gk in GRADS.items():
        fd = _fd(c, w, key, softplus)
        np.testing.assert_allclose(g[gk], fd, rtol=1e-6, atol=1e-7 * np.max(np.abs(fd)),
                                   err_msg=key)


def test_gradients_without_optional_inputs():
    c, w = _case(201, gate=False, h0=False, bias=False, D=False)
    w["dlast"] = np.zeros_like(w["dlast"])
    g = oracle.scan_bwd(**c, **w)
    assert set(g) == {"du", "ddelta", "dA", "dB", "dC"}
    for key in ("u", "delta", "A", "B", "C"):
        fd = _fd(c, w, key)
        np.testing.assert_allclose(g[GRADS[key]], fd, rtol=1e-6,
                                   atol=1e-7 * np.max(np.abs(fd)), err_msg=key)


def test_integrator_closed_form():
    """N = 1, A = 0, softplus off, no D, no gate: h_t = sum_{s<=t} Delta_s u_s B_s
    and y_t = C_t h_t, so dL/du_s = Delta_s B_s sum_{t>=s} w_t C_t,
    dL/dC_t = w_t h_t and dL/dDelta_s = u_s B_s sum_{t>=s} w_t C_t."""
    r = np.random.default_rng(202)
    L = 11
    u = r.standard_normal((1, L, 1))
    dl = r.uniform(0.1, 1.0, (1, L, 1))
    B = r.standard_normal((1, L, 1))
    C = r.standard_normal((1, L, 1))
    wt = r.standard_normal((1, L, 1))
    g = oracle.scan_bwd(u, dl, np.zeros((1, 1)), B, C, delta_softplus=False, dout=wt)
    tail = np.cumsum((wt * C)[0, ::-1, 0])[::-1]                   # sum_{t>=s} w_t C_t
    np.testing.assert_allclose(g["du"][0, :, 0], dl[0, :, 0] * B[0, :, 0] * tail, rtol=1e-13)
    h = np.cumsum((dl * u * B)[0, :, 0])
    np.testing.assert_allclose(g["dC"][0, :, 0], wt[0, :, 0] * h, rtol=1e-13)
    np.testing.assert_allclose(g["ddelta"][0, :, 0], u[0, :, 0] * B[0, :, 0] * tail, rtol=1e-13)
    # dA = sum_t lambda_t h_{t-1} Delta_t with lambda_t = tail_t (Abar = 1)
    h_prev = np.concatenate([[0.0], h[:-1]])
    np.testing.assert_allclose(g["dA"][0, 0], np.sum(tail * h_prev * dl[0, :, 0]), rtol=1e-13)


def test_final_state_gradient_alone():
    """dout = 0, dlast = e_k: the loss is the final state h_{L-1}[k], and with
    softplus off and no input (u = 0) h_{L-1} = prod_t Abar_t h0, so
    dL/dh0 = prod_t exp(Delta_t A) and dL/dA = h_{L-1} * sum_t Delta_t."""
    r = np.random.default_rng(203)
    L, d, n = 7, 2, 3
    dl = r.uniform(0.1, 0.5, (1, L, d))
    A = -r.uniform(0.5, 2.0, (d, n))
    h0 = r.standard_normal((1, d, n))
    dlast = np.zeros((1, d, n))
    dlast[0, 1, 2] = 1.0
    g = oracle.scan_bwd(np.zeros((1, L, d)), dl, A, r.standard_normal((1, L, n)),
                        r.standard_normal((1, L, n)), delta_softplus=False, h0=h0,
                        dout=np.zeros((1, L, d)), dlast=dlast)
    T = dl[0, :, 1].sum()
    hL = np.exp(A[1, 2] * T) * h0[0, 1, 2]
    assert abs(g["dh0"][0, 1, 2] - np.exp(A[1, 2] * T)) <= 1e-14
    assert abs(g["dA"][1, 2] - hL * T) <= 1e-13 * max(1.0, abs(hL * T))
    mask = np.ones((d, n), bool)
    mask[1, 2] = False
    assert np.all(g["dA"][mask] == 0.0)
    assert np.all(g["dh0"][0][mask] == 0.0)


# ---------------------------------------------------- exact zero-order hold --

def _loss_zoh(c, w, softplus=True):
    out, last = oracle.scan_fwd(**c, delta_softplus=softplus, bbar="zoh")
    return float(np.sum(out * w["dout"]) + np.sum(last * w["dlast"]))


def _fd_zoh(c, w, key, softplus=True, eps=1e-6):
    x = c[key]
    g = np.empty_like(x)
    for i in np.ndindex(x.shape):
        cp = dict(c)
        xp = x.copy()
        xp[i] += eps
        cp[key] = xp
        lp = _loss_zoh(cp, w, softplus)
        xp[i] -= 2 * eps
        lm = _loss_zoh(cp, w, softplus)
        g[i] = (lp - lm) / (2 * eps)
    return g


@pytest.mark.parametrize("softplus", [True, False])
def test_zoh_gradients_match_finite_differences(softplus):
    """The ZOH input (reading guide, Method): every gradient against central
    differences of the forward oracle in its ZOH mode."""
    c, w = _case(210, gate=True, h0=True)
    if not softplus:
        c["delta"] = np.abs(c["delta"]) * 0.3
        c["dt_bias"] = np.full(3, 0.05)
    g = oracle.scan_bwd(**c, delta_softplus=softplus, bbar="zoh", **w)
    for key, gk in GRADS.items():
        fd = _fd_zoh(c, w, key, softplus)
        np.testing.assert_allclose(g[gk], fd, rtol=1e-6, atol=1e-7 * np.max(np.abs(fd)),
                                   err_msg=key)


def test_zoh_gradients_near_zero_A():
    """A at 0 and within 1e-4 of it, where (exp(Delta A) - 1)/A and its
    derivative in A take their series forms."""
    c, w = _case(211, gate=False, h0=True)
    c["A"][0, 0] = 0.0
    c["A"][1, 1] = -1e-7
    c["A"][2, 2] = -3e-5
    c["A"][0, 3] = 2e-6
    g = oracle.scan_bwd(**c, bbar="zoh", **w)
    for key in ("A", "delta", "u", "B"):
        fd = _fd_zoh(c, w, key)
        np.testing.assert_allclose(g[GRADS[key]], fd, rtol=1e-6,
                                   atol=1e-7 * np.max(np.abs(fd)), err_msg=key)


def test_zoh_gated_rnn_input_gradient():
    """N = 1, A = -1, B = C = 1: the ZOH step is h_t = (1 - g_t) h_{t-1} + g_t x_t
    with g_t = sigmoid(s_t) (reading guide, S6's gated-RNN special case), so
    the final state's gradient in x_t is g_t prod_{r>t} (1 - g_r)."""
    r = np.random.default_rng(212)
    L = 6
    s = r.standard_normal((1, L, 1))
    x = r.standard_normal((1, L, 1))
    g = oracle.scan_bwd(x, s, -np.ones((1, 1)), np.ones((1, L, 1)), np.ones((1, L, 1)),
                        dout=np.zeros((1, L, 1)), dlast=np.ones((1, 1, 1)), bbar="zoh")
    gate = 1.0 / (1.0 + np.exp(-s[0, :, 0]))
    want = np.array([gate[t] * np.prod(1.0 - gate[t + 1:]) for t in range(L)])
    np.testing.assert_allclose(g["du"][0, :, 0], want, rtol=1e-13)
