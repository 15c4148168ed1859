"""Pins of the oracle's segment carry record and carry combination.

A sequence cut into segments is scanned by composing each segment's steps
into one transform ("Mamba / MambaMini", Steps 2-4): a record of the sum of
Delta (the decay product is exp(A * sum Delta) because A is time-invariant)
and the state reached from zero.  The expectations below come from the
brute-force closed form of the recurrence, written out here with explicit
products, and from library routines (numpy.logaddexp for softplus), never
from the oracle function under test.
"""

import numpy as np
import pytest

import oracle


def _case(seed, b=2, L=23, d=5, n=4):
    r = np.random.default_rng(seed)
    return dict(
        u=r.standard_normal((b, L, d)),
        delta=r.standard_normal((b, L, d)),
        A=-np.exp(r.standard_normal((d, n))),
        B=r.standard_normal((b, L, n)),
        dt_bias=r.uniform(-4.0, -1.0, d),
        h0=r.standard_normal((b, d, n)),
    )


def _deltas(c):
    # softplus(s) = log(e^0 + e^s), a library routine
    return np.logaddexp(0.0, c["delta"] + c["dt_bias"])


def _inputs(c, dl, bbar):
    """Bbar_t x_t for every step, [b, L, d, n], written out from its definition."""
    if bbar == "delta":
        return (dl * c["u"])[..., None] * c["B"][:, :, None, :]
    x = dl[..., None] * c["A"]
    return (np.expm1(x) / c["A"]) * c["B"][:, :, None, :] * c["u"][..., None]


def _closed_form_state(c, dl, bbar, t_end, h0):
    """h after step t_end - 1 = sum_s (prod_{s<r<t_end} Abar_r) Bbar_s x_s
    + (prod_{r<t_end} Abar_r) h0, by explicit products (O(L^2))."""
    abar = np.exp(dl[..., None] * c["A"])
    bx = _inputs(c, dl, bbar)
    h = np.zeros(c["h0"].shape)
    for s in range(t_end):
        p = np.ones_like(h)
        for r in range(s + 1, t_end):
            p = p * abar[:, r]
        h = h + p * bx[:, s]
    if h0 is not None:
        p = np.ones_like(h)
        for r in range(t_end):
            p = p * abar[:, r]
        h = h + p * h0
    return h


@pytest.mark.parametrize("bbar", ["delta", "zoh"])
@pytest.mark.parametrize("with_h0", [False, True])
def test_aggregate_state_matches_closed_form(bbar, with_h0):
    """The record's state is the recurrence's end state (Step 4: h = A_cum h0
    + B_cum; B_cum alone from a zero start)."""
    c = _case(1)
    dl = _deltas(c)
    h0 = c["h0"] if with_h0 else None
    sd, st = oracle.segment_aggregate(c["u"], c["delta"], c["A"], c["B"], dt_bias=c["dt_bias"],
                                      h0=h0, bbar=bbar)
    want = _closed_form_state(c, dl, bbar, dl.shape[1], h0)
    np.testing.assert_allclose(st, want, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sd, dl.sum(axis=1), rtol=1e-13)


def test_sum_delta_closed_forms():
    """dt + bias = 0 gives Delta = softplus(0) = ln 2 at every step; without
    softplus, small integers sum exactly."""
    r = np.random.default_rng(2)
    b, L, d, n = 1, 12, 3, 2
    bias = np.array([-1.0, 0.5, 2.0])
    dt = np.broadcast_to(-bias, (b, L, d)).copy()
    sd, _ = oracle.segment_aggregate(r.standard_normal((b, L, d)), dt, -np.ones((d, n)),
                                     r.standard_normal((b, L, n)), dt_bias=bias)
    np.testing.assert_allclose(sd, np.full((b, d), L * np.log(2.0)), rtol=1e-14)
    dti = r.integers(-3, 4, (b, L, d)).astype(np.float64)
    sd2, _ = oracle.segment_aggregate(np.ones((b, L, d)), dti, -np.ones((d, n)),
                                      np.ones((b, L, n)), delta_softplus=False)
    assert np.array_equal(sd2, dti.sum(axis=1))


def test_decay_product_is_exp_of_sum():
    """prod_t exp(Delta_t A) = exp(A sum_t Delta_t): the one number per channel
    that stands for the segment's decay (A time-invariant, reading guide
    Method; "Mamba / MambaMini" Q&A: A has no time index)."""
    c = _case(3, L=40)
    sd, _ = oracle.segment_aggregate(c["u"], c["delta"], c["A"], c["B"], dt_bias=c["dt_bias"])
    prod = np.prod(np.exp(_deltas(c)[..., None] * c["A"]), axis=1)
    np.testing.assert_allclose(np.exp(sd[..., None] * c["A"]), prod, rtol=1e-12)


@pytest.mark.parametrize("bbar", ["delta", "zoh"])
@pytest.mark.parametrize("cuts", [(7,), (3, 11, 12, 20), (1, 2, 22)])
def test_combined_records_give_every_segment_start(bbar, cuts):
    """Records of consecutive segments (each from a zero start), folded with
    the pair operator from h0, give every segment's true start state and the
    sequence's end state (Steps 2-4), checked against the closed form."""
    c = _case(4)
    dl = _deltas(c)
    L = dl.shape[1]
    bounds = [0, *cuts, L]
    sds, aggs = [], []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        sd, st = oracle.segment_aggregate(c["u"][:, lo:hi], c["delta"][:, lo:hi], c["A"],
                                          c["B"][:, lo:hi], dt_bias=c["dt_bias"], bbar=bbar)
        sds.append(sd)
        aggs.append(st)
    h_in, h_out = oracle.carry_combine(np.stack(sds), np.stack(aggs), c["A"], h0=c["h0"])
    for s, lo in enumerate(bounds[:-1]):
        np.testing.assert_allclose(h_in[s], _closed_form_state(c, dl, bbar, lo, c["h0"]),
                                   rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(h_out, _closed_form_state(c, dl, bbar, L, c["h0"]),
                               rtol=1e-11, atol=1e-12)


def test_combine_without_initial_state():
    """With no h0, segment 0 starts from zero and the end state is the whole
    sequence's B_cum."""
    c = _case(5)
    dl = _deltas(c)
    half = dl.shape[1] // 2
    recs = [oracle.segment_aggregate(c["u"][:, a:b_], c["delta"][:, a:b_], c["A"],
                                     c["B"][:, a:b_], dt_bias=c["dt_bias"])
            for a, b_ in ((0, half), (half, dl.shape[1]))]
    h_in, h_out = oracle.carry_combine(np.stack([r[0] for r in recs]),
                                       np.stack([r[1] for r in recs]), c["A"])
    assert np.array_equal(h_in[0], np.zeros_like(h_in[0]))
    np.testing.assert_allclose(h_in[1], _closed_form_state(c, dl, "delta", half, None),
                               rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(h_out, _closed_form_state(c, dl, "delta", dl.shape[1], None),
                               rtol=1e-11, atol=1e-12)
