"""Pin of the oracle's Mamba block (oracle.block) against a brute-force
scalar evaluation written independently of it: explicit loops over tokens,
channels and states, no vectorised helper shared with the oracle (reading
guide glossary "Mamba Block"; "Mamba / MambaMini" Q&A on the projections,
the Conv and the low-rank Delta)."""

import math

import numpy as np

import oracle


def _weights(r, dm, di, n, rank, k):
    s = 1.0 / math.sqrt(dm)
    return dict(
        in_x=r.standard_normal((dm, di)) * s, in_z=r.standard_normal((dm, di)) * s,
        conv_w=r.standard_normal((di, k)) * 0.5, conv_b=r.standard_normal(di) * 0.1,
        x_dt=r.standard_normal((di, rank)) / math.sqrt(di),
        x_B=r.standard_normal((di, n)) / math.sqrt(di),
        x_C=r.standard_normal((di, n)) / math.sqrt(di),
        dt=r.standard_normal((rank, di)) / math.sqrt(rank),
        dt_bias=np.log(np.expm1(r.uniform(1e-3, 1e-1, di))),
        A=-np.exp(r.standard_normal((di, n))), D=r.standard_normal(di),
        out=r.standard_normal((di, dm)) / math.sqrt(di))


def _brute(x_in, w):
    b_, L, dm = x_in.shape
    di, k = w["conv_w"].shape
    n = w["A"].shape[1]
    rank = w["dt"].shape[0]
    sig = lambda v: 1.0 / (1.0 + math.exp(-v))
    out = np.zeros((b_, L, dm))
    for b in range(b_):
        xs = [[sum(x_in[b, t, m] * w["in_x"][m, d] for m in range(dm)) for d in range(di)]
              for t in range(L)]
        zs = [[sum(x_in[b, t, m] * w["in_z"][m, d] for m in range(dm)) for d in range(di)]
              for t in range(L)]
        h = [[0.0] * n for _ in range(di)]
        for t in range(L):
            u = []
            for d in range(di):
                a = w["conv_b"][d]
                for j in range(k):
                    tt = t - (k - 1) + j
                    if tt >= 0:
                        a += w["conv_w"][d, j] * xs[tt][d]
                u.append(a * sig(a))
            low = [sum(u[d] * w["x_dt"][d, q] for d in range(di)) for q in range(rank)]
            Bt = [sum(u[d] * w["x_B"][d, q] for d in range(di)) for q in range(n)]
            Ct = [sum(u[d] * w["x_C"][d, q] for d in range(di)) for q in range(n)]
            y = []
            for d in range(di):
                s = sum(low[q] * w["dt"][q, d] for q in range(rank)) + w["dt_bias"][d]
                delta = math.log1p(math.exp(s)) if s < 30 else s
                acc = 0.0
                for q in range(n):
                    h[d][q] = math.exp(delta * w["A"][d, q]) * h[d][q] + delta * Bt[q] * u[d]
                    acc += Ct[q] * h[d][q]
                acc += w["D"][d] * u[d]
                zz = zs[t][d]
                y.append(acc * zz * sig(zz))
            for m in range(dm):
                out[b, t, m] = sum(y[d] * w["out"][d, m] for d in range(di))
    return out


def test_block_matches_brute_force():
    r = np.random.default_rng(400)
    dm, di, n, rank, k = 3, 6, 4, 2, 4
    w = _weights(r, dm, di, n, rank, k)
    x_in = r.standard_normal((2, 9, dm))
    got = oracle.mamba_block_fwd(x_in, w)
    ref = _brute(x_in, w)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12 * np.max(np.abs(ref)))


def test_block_is_causal():
    """Changing token t leaves every earlier output unchanged (conv and scan
    are both causal)."""
    r = np.random.default_rng(401)
    w = _weights(r, 4, 8, 4, 2, 4)
    x_in = r.standard_normal((1, 12, 4))
    o1 = oracle.mamba_block_fwd(x_in, w)
    x2 = x_in.copy()
    x2[0, 7] += 1.0
    o2 = oracle.mamba_block_fwd(x2, w)
    assert np.array_equal(o1[0, :7], o2[0, :7])
    assert not np.allclose(o1[0, 7:], o2[0, 7:])
