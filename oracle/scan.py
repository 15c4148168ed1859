"""Plain float64 reference of the selective scan (S6) and its decode step.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Shapes and layouts:

    u, delta, z   [batch, L, dim]      token-major activations
    A             [dim, dstate]        time-invariant, negative in practice
    B, C          [batch, L, dstate]   input-dependent, shared by all channels
    D, dt_bias    [dim]
    h0, state     [batch, dim, dstate]

Inputs of any float dtype are widened to float64 first, which is exact for
float32 and bfloat16 values, so the oracle's only rounding is float64's.
"""

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def softplus(s):
    """softplus(s) = log(1 + e^s), the positive activation that turns the raw
    step into Delta.

    Gu & Dao reading guide, "Selection mechanism (S6)": Delta is tau_Delta of
    (Parameter + s_Delta(x)) with tau_Delta = softplus.  Written in the
    overflow-free form max(s, 0) + log1p(exp(-|s|)), which is the same
    function for every real s.
    """
    s = _f64(s)
    return np.maximum(s, 0.0) + np.log1p(np.exp(-np.abs(s)))


def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^-z).

    "Mamba / MambaMini", Q&A on why the gate activation is SiLU: it defines
    Sigmoid(x) = 1/(1+exp(-x)) and SiLU(x) = x * Sigmoid(x).
    """
    z = _f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def combine(later, earlier):
    """The pair operator of the parallel scan.

    "Mamba / MambaMini", Step 2: applying T_i then T_j (j = i + 1) equals the
    single transform T_j (+) T_i = (a_j * a_i, a_j * b_i + b_j).  ``later``
    and ``earlier`` are (a, b) tuples of broadcastable arrays.
    """
    a_j, b_j = later
    a_i, b_i = earlier
    return a_j * a_i, a_j * b_i + b_j


def discretise(delta, A, B_t, u_t, bbar="delta"):
    """Per-step discretisation for one time step.

    delta, u_t: [..., dim]; A: [dim, dstate]; B_t: [..., dstate].
    Returns (Abar, Bbar*x), each [..., dim, dstate].

    Abar = exp(Delta * A): Gu & Dao reading guide, "Method" (zero-order hold).
    Bbar * x:
      * bbar="delta": Delta * B * x, the simplified input discretisation of
        "Mamba / MambaMini" Q&A (Delta multiplies B elementwise).  The
        default of the GPU entry points.
      * bbar="zoh": the exact ZOH input matrix of the reading guide's
        "Method", (Delta A)^-1 (exp(Delta A) - 1) Delta B, which for diagonal
        A is expm1(Delta A) / A * B (limit Delta * B as A -> 0).  The GPU's
        optional zero-order-hold mode.
    """
    dA = delta[..., :, None] * A
    Abar = np.exp(dA)
    if bbar == "delta":
        bx = (delta * u_t)[..., :, None] * B_t[..., None, :]
    elif bbar == "zoh":
        with np.errstate(divide="ignore", invalid="ignore"):
            coef = np.where(A == 0.0, delta[..., :, None], np.expm1(dA) / A)
        bx = coef * B_t[..., None, :] * u_t[..., :, None]
    else:
        raise ValueError(bbar)
    return Abar, bx


def _delta(dt_t, dt_bias, use_softplus):
    s = dt_t if dt_bias is None else dt_t + dt_bias
    return softplus(s) if use_softplus else s


def _step(h, u_t, dt_t, A, B_t, C_t, D, z_t, dt_bias, use_softplus, bbar):
    """One step of the recurrence and readout for all (batch, channel).

    h_t = Abar_t * h_{t-1} + Bbar_t x_t and y_t = C_t . h_t + D x_t
    (reading guide "Method"; the D term is the direct input-to-output path of
    the CSDN tutorial, section 3(1)).  The readout uses the updated state h_t.
    The gate multiplies y by SiLU(z) ("Mamba / MambaMini" Q&A on SiLU; the
    reading guide's "Mamba Block" glossary entry on multiplicative gating).
    """
    delta = _delta(dt_t, dt_bias, use_softplus)
    Abar, bx = discretise(delta, A, B_t, u_t, bbar)
    h = Abar * h + bx
    y = np.sum(h * C_t[..., None, :], axis=-1)
    if D is not None:
        y = y + D * u_t
    if z_t is not None:
        y = y * silu(z_t)
    return h, y


def scan_fwd(u, delta, A, B, C, D=None, z=None, dt_bias=None,
             delta_softplus=True, h0=None, bbar="delta", return_states=False):
    """Selective-scan forward: the sequential recurrence over the sequence.

    The parallel scan of "Mamba / MambaMini" (Steps 1-4) only re-associates
    the pair operator, so its result is exactly this serial loop (the
    O(L) "RNN-like" form that the same page uses for clarity).  The initial
    state is h_{-1} = 0 (Step 4) unless ``h0`` is given.

    Returns (out [batch, L, dim], last_state [batch, dim, dstate]) and, with
    ``return_states``, also every state [batch, L, dim, dstate].
    """
    u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
    D, z, dt_bias, h0 = map(_f64, (D, z, dt_bias, h0))
    bsz, L, dim = u.shape
    dstate = A.shape[1]
    h = np.zeros((bsz, dim, dstate)) if h0 is None else h0.copy()
    out = np.empty((bsz, L, dim))
    states = np.empty((bsz, L, dim, dstate)) if return_states else None
    for t in range(L):
        h, y = _step(h, u[:, t], delta[:, t], A, B[:, t], C[:, t], D,
                     None if z is None else z[:, t], dt_bias, delta_softplus,
                     bbar)
        out[:, t] = y
        if return_states:
            states[:, t] = h
    if return_states:
        return out, h, states
    return out, h


def state_update(state, x, dt, A, B, C, D=None, z=None, dt_bias=None,
                 dt_softplus=True, bbar="delta"):
    """Single-token decode: one step of the same recurrence on a stored state.

    Reading guide FAQ (no KV cache): generation keeps only a fixed D x N state
    per layer and advances it once per token.  state [batch, dim, dstate];
    x, dt, z [batch, dim]; B, C [batch, dstate].
    Returns (out [batch, dim], new_state [batch, dim, dstate]).
    """
    state, x, dt, A, B, C = map(_f64, (state, x, dt, A, B, C))
    D, z, dt_bias = map(_f64, (D, z, dt_bias))
    h, y = _step(state, x, dt, A, B, C, D, z, dt_bias, dt_softplus, bbar)
    return y, h


def scan_pairs_blelloch(a, b):
    """Inclusive prefix of the pairs (a_t, b_t) along the last axis with the
    work-efficient up-sweep / down-sweep scan.

    "Mamba / MambaMini", Step 4: the up-sweep builds a tree of interval
    combinations, the down-sweep pushes prefixes back down; the prefix
    S_t = T_t (+) ... (+) T_0 = (A_cum_t, B_cum_t) gives
    h_t = A_cum_t * h_{-1} + B_cum_t.  The CSDN tutorial, section (2)(2),
    names the same Blelloch scan.  Serves as an independent cross-check of the
    serial loop; the operator is not commutative, so the later element is
    always the left operand of ``combine``.
    """
    a = _f64(a)
    b = _f64(b)
    L = a.shape[-1]
    n = 1
    while n < L:
        n *= 2
    pad = [(0, 0)] * (a.ndim - 1) + [(0, n - L)]
    xa = np.pad(a, pad, constant_values=1.0)   # identity element (1, 0)
    xb = np.pad(b, pad, constant_values=0.0)
    oa, ob = xa.copy(), xb.copy()
    # up-sweep: node k+2d1-1 becomes (right subtree) (+) (left subtree)
    d = 1
    while d < n:
        d1 = 2 * d
        for k in range(0, n, d1):
            r, l_ = k + d1 - 1, k + d - 1
            xa[..., r], xb[..., r] = combine((xa[..., r], xb[..., r]),
                                             (xa[..., l_], xb[..., l_]))
        d = d1
    # down-sweep for the exclusive prefix; the root gets the identity
    xa[..., n - 1] = 1.0
    xb[..., n - 1] = 0.0
    d = n // 2
    while d >= 1:
        d1 = 2 * d
        for k in range(0, n, d1):
            r, l_ = k + d1 - 1, k + d - 1
            left_a, left_b = xa[..., l_].copy(), xb[..., l_].copy()
            par_a, par_b = xa[..., r].copy(), xb[..., r].copy()
            # left child inherits the parent's prefix; the right child sees
            # the left subtree applied after that prefix
            xa[..., l_], xb[..., l_] = par_a, par_b
            xa[..., r], xb[..., r] = combine((left_a, left_b), (par_a, par_b))
        d //= 2
    # inclusive = own element applied after the exclusive prefix
    ia, ib = combine((oa, ob), (xa, xb))
    return ia[..., :L], ib[..., :L]


def segment_aggregate(u, delta, A, B, dt_bias=None, delta_softplus=True, h0=None,
                      bbar="delta"):
    """Carry record of one sequence segment: its sum of Delta and its end state.

    "Mamba / MambaMini", Steps 2-4: the steps of a segment compose under the
    pair operator into one transform (A_cum, B_cum), and the state after the
    segment is A_cum * h_start + B_cum.  A is time-invariant, so the product
    of the per-step decays exp(Delta_t A) is exp(A * sum_t Delta_t): a
    segment's A_cum is carried by one number per (batch, channel).  B_cum is
    the state the segment reaches from h_start = 0.

    Returns (sum_delta [batch, dim], state [batch, dim, dstate]) where
    ``state`` is the state after the last step starting from ``h0`` (zeros
    when None, which makes it B_cum).  No readout is formed.
    """
    u, delta, A, B = map(_f64, (u, delta, A, B))
    dt_bias, h0 = map(_f64, (dt_bias, h0))
    bsz, L, dim = u.shape
    h = np.zeros((bsz, dim, A.shape[1])) if h0 is None else h0.copy()
    total = np.zeros((bsz, dim))
    for t in range(L):
        dl = _delta(delta[:, t], dt_bias, delta_softplus)
        Abar, bx = discretise(dl, A, B[:, t], u[:, t], bbar)
        h = Abar * h + bx
        total = total + dl
    return total, h


def carry_combine(sum_delta, agg, A, h0=None):
    """Start state of every segment of a sequence from the segments' records.

    ``sum_delta`` [S, batch, dim] and ``agg`` [S, batch, dim, dstate] are the
    records of S consecutive segments (each ``agg`` from a zero start).  The
    start of segment 0 is h0 (zeros when None); segment s + 1 starts from
    segment s's transform (exp(A sum_delta[s]), agg[s]) applied to segment s's
    start: the exclusive prefix of the pair operator over the segment index
    ("Mamba / MambaMini", Steps 2 and 4), folded in sequence order.

    Returns (h_in [S, batch, dim, dstate], h_out [batch, dim, dstate]), h_out
    being the state after the last segment.
    """
    sum_delta, agg, A, h0 = map(_f64, (sum_delta, agg, A, h0))
    S = agg.shape[0]
    h = np.zeros(agg.shape[1:]) if h0 is None else h0.copy()
    h_in = np.empty(agg.shape)
    for s in range(S):
        h_in[s] = h
        a = np.exp(sum_delta[s][..., None] * A)
        _, h = combine((a, agg[s]), (np.ones_like(h), h))
    return h_in, h
