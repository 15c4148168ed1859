"""Pins of the oracle's causal depthwise conv1d + SiLU (oracle.conv1d)
against numpy's convolution, the impulse response, closed forms of the
activation, and the state hand-off ("Mamba / MambaMini" Q&A on the Conv before
the SSM; reading guide glossary "Mamba Block")."""

import numpy as np
import pytest
from scipy.special import expit

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_equals_numpy_convolve(k):
    r = _rng(300 + k)
    b, L, d = 2, 23, 5
    x = r.standard_normal((b, L, d))
    w = r.standard_normal((d, k))
    out, _ = oracle.causal_conv1d(x, w, activation=None)
    for bi in range(b):
        for di in range(d):
            ref = np.convolve(x[bi, :, di], w[di, ::-1])[:L]
            np.testing.assert_allclose(out[bi, :, di], ref, rtol=1e-13, atol=1e-14)


def test_impulse_response_is_reversed_filter():
    k, L = 4, 12
    w = np.array([[0.5, -1.25, 2.0, 3.5]])
    x = np.zeros((1, L, 1))
    x[0, 5, 0] = 1.0
    out, _ = oracle.causal_conv1d(x, w, activation=None)
    expect = np.zeros(L)
    expect[5:5 + k] = w[0, ::-1]
    assert np.array_equal(out[0, :, 0], expect)


def test_width_one_bias_and_silu_closed_form():
    r = _rng(310)
    x = r.standard_normal((3, 7, 4))
    w = r.standard_normal((4, 1))
    bias = r.standard_normal(4)
    out, final = oracle.causal_conv1d(x, w, bias)
    a = w[:, 0] * x + bias
    np.testing.assert_allclose(out, a * expit(a), rtol=1e-14, atol=1e-300)
    assert final.shape == (3, 4, 0)


@pytest.mark.parametrize("k", [2, 3, 4])
def test_state_hand_off_and_decode_bitwise(k):
    r = _rng(320 + k)
    b, L, d = 2, 19, 6
    x = r.standard_normal((b, L, d))
    w = r.standard_normal((d, k))
    bias = r.standard_normal(d)
    s0 = r.standard_normal((b, d, k - 1))
    out, final = oracle.causal_conv1d(x, w, bias, init_state=s0)
    # the final state is the last K-1 inputs, oldest first
    assert np.array_equal(final, np.transpose(x[:, L - (k - 1):], (0, 2, 1)))
    # split the sequence, carrying the state
    for L1 in (1, k - 1, 7):
        o1, f1 = oracle.causal_conv1d(x[:, :L1], w, bias, init_state=s0)
        o2, f2 = oracle.causal_conv1d(x[:, L1:], w, bias, init_state=f1)
        assert np.array_equal(np.concatenate([o1, o2], axis=1), out)
        assert np.array_equal(f2, final)
    # token by token
    st = s0.copy()
    for t in range(L):
        y, st = oracle.conv1d_update(st, x[:, t], w, bias)
        assert np.array_equal(y, out[:, t])
    assert np.array_equal(st, final)


def test_short_sequence_state_mixes_initial_state():
    k = 4
    x = np.arange(1.0, 3.0).reshape(1, 2, 1)          # two inputs: 1, 2
    s0 = np.array([[[10.0, 20.0, 30.0]]])
    _, final = oracle.causal_conv1d(x, np.ones((1, k)), init_state=s0)
    assert np.array_equal(final[0, 0], [30.0, 1.0, 2.0])
