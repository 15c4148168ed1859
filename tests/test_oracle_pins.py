"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test names the passage it relies on.  None of them re-calls the oracle
to produce its own expectation: expectations come from closed forms, brute
force, library routines (numpy.convolve, scipy.special) or hand arithmetic.
"""

import json
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _random_case(seed, b=2, L=17, d=5, n=4, gate=True, h0=False):
    r = _rng(seed)
    case = dict(
        u=r.standard_normal((b, L, d)),
        delta=r.standard_normal((b, L, d)),
        A=-np.exp(r.standard_normal((d, n))),
        B=r.standard_normal((b, L, n)),
        C=r.standard_normal((b, L, n)),
        D=r.standard_normal(d),
        z=r.standard_normal((b, L, d)) if gate else None,
        dt_bias=r.uniform(-4, -1, d),
    )
    if h0:
        case["h0"] = r.standard_normal((b, d, n))
    return case


# --- P1: the pair operator is associative ("Mamba / MambaMini", Step 3) ----

def test_combine_associative_random():
    r = _rng(1)
    T = [(r.uniform(0, 1, 1000), r.standard_normal(1000)) for _ in range(3)]
    k, j, i = T
    left = oracle.combine(oracle.combine(k, j), i)
    right = oracle.combine(k, oracle.combine(j, i))
    scale = 1 + np.abs(left[1])
    assert np.max(np.abs(left[0] - right[0])) <= 1e-15
    assert np.max(np.abs(left[1] - right[1]) / scale) <= 1e-14


def test_combine_associative_small_integers_bitwise():
    vals = np.arange(-3, 4, dtype=np.float64)
    g = np.array(np.meshgrid(*([vals] * 6), indexing="ij")).reshape(6, -1)
    k, j, i = (g[0], g[1]), (g[2], g[3]), (g[4], g[5])
    left = oracle.combine(oracle.combine(k, j), i)
    right = oracle.combine(k, oracle.combine(j, i))
    assert np.array_equal(left[0], right[0])
    assert np.array_equal(left[1], right[1])


def test_combine_order_is_later_on_left():
    # Step 2: applying T_i then T_j gives (a_j a_i, a_j b_i + b_j).
    a_i, b_i, a_j, b_j, h = 0.5, 3.0, 0.25, -1.0, 7.0
    two_steps = a_j * (a_i * h + b_i) + b_j
    a, b = oracle.combine((a_j, b_j), (a_i, b_i))
    assert a * h + b == two_steps


# --- P2: serial recurrence == brute-force closed form == Blelloch scan -----

def _closed_form_states(Abar, bx, h0):
    """h_t = sum_{s<=t} (prod_{s<r<=t} Abar_r) bx_s + (prod_{r<=t} Abar_r) h0,
    evaluated term by term (O(L^2))."""
    L = Abar.shape[1]
    out = np.zeros_like(bx)
    for t in range(L):
        acc = np.prod(Abar[:, : t + 1], axis=1) * h0
        for s in range(t + 1):
            acc = acc + np.prod(Abar[:, s + 1: t + 1], axis=1) * bx[:, s]
        out[:, t] = acc
    return out


@pytest.mark.parametrize("seed,L,n,h0", [(2, 1, 1, False), (3, 9, 4, False),
                                         (4, 23, 3, True), (5, 32, 16, True)])
def test_recurrence_matches_closed_form(seed, L, n, h0):
    c = _random_case(seed, b=2, L=L, d=3, n=n, gate=True, h0=h0)
    out, last, states = oracle.scan_fwd(**c, return_states=True)
    # discretisation written out from its definition (reading guide, Method)
    dlt = np.logaddexp(0.0, c["delta"] + c["dt_bias"])            # softplus
    Abar = np.exp(dlt[..., None] * c["A"])                         # [b,L,d,n]
    bx = (dlt * c["u"])[..., None] * c["B"][:, :, None, :]
    h0v = c["h0"] if h0 else np.zeros((2, 3, n))
    ref_states = _closed_form_states(Abar, bx, h0v)
    scale = np.max(np.abs(ref_states))
    assert np.max(np.abs(states - ref_states)) <= 1e-12 * scale
    assert np.array_equal(last, states[:, -1])
    y = np.einsum("bln,bldn->bld", c["C"], ref_states) + c["D"] * c["u"]
    y = y * c["z"] * expit(c["z"])
    assert np.max(np.abs(out - y)) <= 1e-12 * np.max(np.abs(y))


def test_tiny_workload_matches_closed_form():
    x = synth.make("tiny")
    out, last, states = oracle.scan_fwd(
        x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"],
        x["dt_bias"], return_states=True)
    dlt = np.logaddexp(0.0, x["delta"].astype(np.float64) + x["dt_bias"])
    Abar = np.exp(dlt[..., None] * x["A"].astype(np.float64))
    bx = (dlt * x["u"])[..., None] * x["B"][:, :, None, :].astype(np.float64)
    ref = _closed_form_states(Abar, bx, np.zeros((1, 16, 4)))
    assert np.max(np.abs(states - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("L", [1, 2, 7, 16, 33])
def test_recurrence_matches_blelloch(L):
    r = _rng(10 + L)
    a = r.uniform(0.0, 1.0, (3, L))
    b = r.standard_normal((3, L))
    _, bcum = oracle.scan_pairs_blelloch(a, b)
    # serial loop h_t = a_t h_{t-1} + b_t, written out here
    h = np.zeros(3)
    ser = np.zeros((3, L))
    for t in range(L):
        h = a[:, t] * h + b[:, t]
        ser[:, t] = h
    assert np.max(np.abs(bcum - ser)) <= 1e-13 * (1 + np.max(np.abs(ser)))


def test_blelloch_prefix_applies_to_initial_state():
    # Step 4: h_t = A_cum_t h_{-1} + B_cum_t for any h_{-1}.
    c = _random_case(20, b=1, L=12, d=2, n=3, gate=False, h0=True)
    out, last, states = oracle.scan_fwd(**c, return_states=True)
    dlt = np.logaddexp(0.0, c["delta"] + c["dt_bias"])
    Abar = np.exp(dlt[..., None] * c["A"])
    bx = (dlt * c["u"])[..., None] * c["B"][:, :, None, :]
    acum, bcum = oracle.scan_pairs_blelloch(np.moveaxis(Abar, 1, -1),
                                            np.moveaxis(bx, 1, -1))
    pred = acum * c["h0"][..., None] + bcum
    assert np.max(np.abs(np.moveaxis(pred, -1, 1) - states)) <= 1e-12 * (
        np.max(np.abs(states)))


# --- hand-worked example (tests/golden/hand_worked.json) --------------------

def _load_hand():
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        return json.load(f)


def test_hand_worked_no_softplus():
    g = _load_hand()
    L = len(g["u"])
    out, last, states = oracle.scan_fwd(
        np.array(g["u"]).reshape(1, L, 1),
        np.array(g["delta_values"]).reshape(1, L, 1),
        np.array(g["A"]), np.array(g["B"]).reshape(1, L, 2),
        np.array(g["C"]).reshape(1, L, 2), np.array(g["D"]),
        delta_softplus=False, return_states=True)
    np.testing.assert_allclose(out.ravel(), g["expected_out"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(last.ravel(), g["expected_last_state"], atol=1e-13)
    np.testing.assert_allclose(states.reshape(L, 2), g["expected_states"], atol=1e-13)


def test_hand_worked_softplus_with_bias():
    g = _load_hand()
    L = len(g["u"])
    bias = g["dt_bias_softplus_case"]
    dt = np.log(np.expm1(np.array(g["delta_values"]))) - bias
    out, last = oracle.scan_fwd(
        np.array(g["u"]).reshape(1, L, 1), dt.reshape(1, L, 1),
        np.array(g["A"]), np.array(g["B"]).reshape(1, L, 2),
        np.array(g["C"]).reshape(1, L, 2), np.array(g["D"]),
        dt_bias=np.array([bias]), delta_softplus=True)
    np.testing.assert_allclose(out.ravel(), g["expected_out"], atol=1e-12)
    np.testing.assert_allclose(last.ravel(), g["expected_last_state"], atol=1e-12)


# --- P3: LTI special case == convolution (CSDN tutorial 3(1)<3>; reading
# guide FAQ on FFT convolutions) -------------------------------------------

@pytest.mark.parametrize("seed,L,n", [(30, 40, 4), (31, 64, 16)])
def test_lti_case_is_convolution(seed, L, n):
    r = _rng(seed)
    d = 3
    dt_const = r.uniform(-3, 0, d)
    Bc = r.standard_normal(n)
    Cc = r.standard_normal(n)
    A = -np.exp(r.standard_normal((d, n)))
    u = r.standard_normal((1, L, d))
    delta = np.broadcast_to(dt_const, (1, L, d)).copy()
    B = np.broadcast_to(Bc, (1, L, n)).copy()
    C = np.broadcast_to(Cc, (1, L, n)).copy()
    out, _ = oracle.scan_fwd(u, delta, A, B, C)
    dlt = np.logaddexp(0.0, dt_const)                 # softplus, [d]
    Abar = np.exp(dlt[:, None] * A)                    # [d, n]
    k = np.arange(L)
    K = np.einsum("n,dkn->dk", Cc, Abar[:, None, :] ** k[None, :, None]
                  * (dlt[:, None] * Bc)[:, None, :])   # K_k = C Abar^k Bbar
    for ch in range(d):
        ref = np.convolve(u[0, :, ch], K[ch])[:L]
        assert np.max(np.abs(out[0, :, ch] - ref)) <= 1e-12 * (1 + np.max(np.abs(ref)))


# --- P4: Delta -> 0 keeps the state ("Mamba / MambaMini" Q&A on Delta and A;
# reading guide FAQ: small Delta persists the state) -------------------------

def test_zero_delta_keeps_state_bitwise():
    c = _random_case(40, b=2, L=11, d=4, n=5, gate=True, h0=True)
    c["delta"] = np.zeros_like(c["delta"])
    c["dt_bias"] = np.zeros_like(c["dt_bias"])
    out, last = oracle.scan_fwd(**c, delta_softplus=False)
    assert np.array_equal(last, c["h0"])
    y = np.einsum("bln,bdn->bld", c["C"], c["h0"]) + c["D"] * c["u"]
    y = y * c["z"] * expit(c["z"])
    assert np.max(np.abs(out - y)) <= 1e-13 * np.max(np.abs(y))
    _, st = oracle.state_update(c["h0"], c["u"][:, 0], c["delta"][:, 0], c["A"],
                                c["B"][:, 0], c["C"][:, 0], dt_softplus=False)
    assert np.array_equal(st, c["h0"])


# --- P5: large Delta resets the state to the current input ("Mamba /
# MambaMini" Q&A: Abar -> 0 forgets history; reading guide FAQ) --------------

def test_large_delta_resets_state():
    c = _random_case(50, b=2, L=9, d=3, n=4, gate=False, h0=True)
    c["A"] = np.minimum(c["A"], -0.1)      # exp(1e4 * A) underflows to 0
    c["delta"] = np.full_like(c["delta"], 1e4)
    c["dt_bias"] = None
    c["D"] = None
    out, last, states = oracle.scan_fwd(**c, delta_softplus=False, return_states=True)
    expect = (1e4 * c["u"])[..., None] * c["B"][:, :, None, :]
    assert np.array_equal(states, expect)


def test_large_delta_resets_state_fixed_A():
    r = _rng(51)
    u = r.standard_normal((1, 6, 2))
    B = r.standard_normal((1, 6, 3))
    C = r.standard_normal((1, 6, 3))
    A = -np.ones((2, 3))
    h0 = r.standard_normal((1, 2, 3))
    delta = np.full((1, 6, 2), 1e4)
    out, last, states = oracle.scan_fwd(u, delta, A, B, C, h0=h0,
                                        delta_softplus=False, return_states=True)
    expect = (1e4 * u)[..., None] * B[:, :, None, :]
    assert np.array_equal(states, expect)
    ref = np.einsum("bln,bldn->bld", C, expect)
    assert np.max(np.abs(out - ref)) <= 1e-13 * np.max(np.abs(ref))


# --- P6: gated-RNN special case (reading guide, Selection mechanism (S6)) ---

def test_gated_rnn_special_case():
    r = _rng(60)
    L = 50
    s = r.normal(0, 2, (1, L, 1))
    x = r.standard_normal((1, L, 1))
    A = -np.ones((1, 1))
    ones = np.ones((1, L, 1))
    # ZOH input matrix: h_t = (1 - g_t) h_{t-1} + g_t x_t with g_t = sigmoid(s_t)
    out_zoh, _, st_zoh = oracle.scan_fwd(x, s, A, ones, ones, bbar="zoh",
                                         return_states=True)
    g = expit(s[0, :, 0])
    h = 0.0
    ref_zoh = []
    for t in range(L):
        h = (1 - g[t]) * h + g[t] * x[0, t, 0]
        ref_zoh.append(h)
    np.testing.assert_allclose(st_zoh[0, :, 0, 0], ref_zoh, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(out_zoh[0, :, 0], ref_zoh, rtol=1e-13, atol=1e-14)
    # simplified input (Delta * B): h_t = sigmoid(-s_t) h_{t-1} + softplus(s_t) x_t
    out_d, _, st_d = oracle.scan_fwd(x, s, A, ones, ones, return_states=True)
    sp = np.logaddexp(0.0, s[0, :, 0])
    h = 0.0
    ref_d = []
    for t in range(L):
        h = expit(-s[0, t, 0]) * h + sp[t] * x[0, t, 0]
        ref_d.append(h)
    np.testing.assert_allclose(st_d[0, :, 0, 0], ref_d, rtol=1e-13, atol=1e-14)


# --- P7: skip term and gate (CSDN tutorial 3(1): D; MambaMini Q&A: SiLU) ----

def test_zero_B_leaves_skip_and_gate():
    c = _random_case(70, b=2, L=8, d=4, n=3, gate=True)
    c["B"] = np.zeros_like(c["B"])
    out, last = oracle.scan_fwd(**c)
    ref = c["D"] * c["u"] * c["z"] * expit(c["z"])
    assert np.max(np.abs(out - ref)) <= 1e-15 * np.max(np.abs(ref)) + 1e-300
    assert np.array_equal(last, np.zeros_like(last))


def test_nullable_skip_gate_bias():
    c = _random_case(71, b=1, L=6, d=3, n=2, gate=False)
    out_none, _ = oracle.scan_fwd(c["u"], c["delta"], c["A"], c["B"], c["C"])
    out_zero, _ = oracle.scan_fwd(c["u"], c["delta"], c["A"], c["B"], c["C"],
                                  D=np.zeros(3), dt_bias=np.zeros(3))
    assert np.array_equal(out_none, out_zero)


# --- P8: linear in u for a zero initial state (Method: linear recurrence) ---

def test_linear_in_input():
    c = _random_case(80, b=2, L=15, d=3, n=4, gate=False)
    u2 = _rng(81).standard_normal(c["u"].shape)
    alpha, beta = 0.7, -1.3
    o1, _ = oracle.scan_fwd(**c)
    c2 = dict(c, u=u2)
    o2, _ = oracle.scan_fwd(**c2)
    c3 = dict(c, u=alpha * c["u"] + beta * u2)
    o3, _ = oracle.scan_fwd(**c3)
    ref = alpha * o1 + beta * o2
    assert np.max(np.abs(o3 - ref)) <= 1e-12 * np.max(np.abs(ref))


# --- P9 / P10: resume from a state; decode equals the forward (Step 4;
# reading guide FAQ on constant-time decoding) -------------------------------

def test_split_resume_bitwise():
    c = _random_case(90, b=2, L=20, d=3, n=4, gate=True)
    out, last = oracle.scan_fwd(**c)
    L1 = 7
    head = {k: (v[:, :L1] if k in ("u", "delta", "B", "C", "z") else v)
            for k, v in c.items()}
    tail = {k: (v[:, L1:] if k in ("u", "delta", "B", "C", "z") else v)
            for k, v in c.items()}
    o1, s1 = oracle.scan_fwd(**head)
    o2, s2 = oracle.scan_fwd(**tail, h0=s1)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), out)
    assert np.array_equal(s2, last)


def test_decode_loop_equals_forward_bitwise():
    c = _random_case(100, b=2, L=10, d=3, n=4, gate=True, h0=True)
    out, last = oracle.scan_fwd(**c)
    st = c["h0"].copy()
    for t in range(10):
        y, st = oracle.state_update(st, c["u"][:, t], c["delta"][:, t], c["A"],
                                    c["B"][:, t], c["C"][:, t], c["D"],
                                    c["z"][:, t], c["dt_bias"])
        assert np.array_equal(y, out[:, t])
    assert np.array_equal(st, last)


# --- P11: columns are independent ("Mamba / MambaMini" Q&A: elementwise) ---

def test_column_independence_bitwise():
    c = _random_case(110, b=3, L=12, d=5, n=4, gate=True)
    out, last = oracle.scan_fwd(**c)
    c2 = {k: (None if v is None else np.array(v, copy=True)) for k, v in c.items()}
    c2["u"][:, :, 2] += 1.0
    c2["delta"][1, :, :] -= 0.5
    c2["z"][:, 3, 2] = 5.0
    out2, last2 = oracle.scan_fwd(**c2)
    keep = np.ones(out.shape, bool)
    keep[:, :, 2] = False
    keep[1] = False
    assert np.array_equal(out[keep], out2[keep])
    keep_s = np.ones(last.shape, bool)
    keep_s[:, 2] = False
    keep_s[1] = False
    assert np.array_equal(last[keep_s], last2[keep_s])


# --- P12: softplus and SiLU helpers against library/closed forms -----------

def test_softplus_closed_forms():
    s = np.array([-50.0, -20.0, 0.0, 20.0, 50.0, 1e-3, -1e-3, 700.0, -700.0])
    got = oracle.softplus(s)
    assert got[2] == np.log(2.0)
    np.testing.assert_allclose(got, np.logaddexp(0.0, s), rtol=1e-15, atol=0)
    assert abs(got[4] - 50.0 - np.exp(-50.0)) <= 1e-13
    assert got[7] == 700.0


def test_silu_closed_form():
    z = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(oracle.silu(z), z * expit(z), rtol=1e-15, atol=1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0


# --- P13: exact zero-order hold (reading guide, Method) ---------------------
# With the input held constant, the ZOH step is the exact solution of
# h' = A h + B x over the step, so steps compose: after any split of a total
# time T into steps Delta_t, h = e^{A T} h0 + (e^{A T} - 1)/A * B x.  The
# simplified Delta*B input does not have this property, so the test also
# tells the two modes apart.

def test_zoh_exact_for_held_input():
    r = _rng(130)
    b, L, d, n = 2, 40, 3, 5
    A = -np.exp(r.normal(0, 2, (d, n)))          # from ~1e-3 to ~50 in size
    A[0, 0] = -1e-9                               # near the A -> 0 limit
    dt = r.uniform(1e-3, 0.2, (b, L, d))          # softplus off: Delta = dt
    Bv = r.standard_normal((b, 1, n))
    x = r.standard_normal((b, 1, d))
    h0 = r.standard_normal((b, d, n))
    u = np.broadcast_to(x, (b, L, d))
    Bm = np.broadcast_to(Bv, (b, L, n))
    C = r.standard_normal((b, L, n))
    _, last = oracle.scan_fwd(u, dt, A, Bm, C, delta_softplus=False, h0=h0, bbar="zoh")
    T = dt.sum(axis=1)[:, :, None]                                  # [b, d, 1]
    decay = np.exp(A[None] * T)
    ref = decay * h0 + np.expm1(A[None] * T) / A[None] * Bv[:, 0, None, :] * x[:, 0, :, None]
    np.testing.assert_allclose(last, ref, rtol=1e-12, atol=1e-13)
    _, last_delta = oracle.scan_fwd(u, dt, A, Bm, C, delta_softplus=False, h0=h0)
    assert np.max(np.abs(last_delta - ref)) > 1e-3 * np.max(np.abs(ref))


def test_zoh_zero_A_is_integrator():
    r = _rng(131)
    b, L, d, n = 1, 12, 2, 3
    A = np.zeros((d, n))
    dt = r.uniform(0.01, 0.5, (b, L, d))
    u = r.standard_normal((b, L, d))
    Bm = r.standard_normal((b, L, n))
    C = r.standard_normal((b, L, n))
    _, last = oracle.scan_fwd(u, dt, A, Bm, C, delta_softplus=False, bbar="zoh")
    ref = np.einsum("bld,bln->bdn", dt * u, Bm)       # h = sum_t Delta_t x_t B_t
    np.testing.assert_allclose(last, ref, rtol=1e-13, atol=1e-14)


def test_zoh_decode_loop_equals_forward_bitwise():
    c = _random_case(132, b=2, L=9, d=3, n=4, gate=True, h0=True)
    out, last = oracle.scan_fwd(**c, bbar="zoh")
    st = c["h0"].copy()
    for t in range(9):
        y, st = oracle.state_update(st, c["u"][:, t], c["delta"][:, t], c["A"],
                                    c["B"][:, t], c["C"][:, t], c["D"],
                                    c["z"][:, t], c["dt_bias"], bbar="zoh")
        assert np.array_equal(y, out[:, t])
    assert np.array_equal(st, last)
