"""GPU parity of the backward (selective_scan_bwd) against the float64
oracle's hand-derived adjoint (oracle.scan_bwd, itself pinned by finite
differences).  Each gradient tensor is held to max-abs error <= tol *
max |oracle gradient| with the forward's tolerances (1e-4 for float32
activations, 2e-2 for bfloat16)."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import TOL, act_dtype, check, env, gpu_available, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _log(msg):
    print(msg, flush=True)


def _grads_in(x, tag, seed, *, dlast=True, h0=True):
    r = np.random.default_rng(seed)
    b, L, d = x["u"].shape
    n = x["A"].shape[1]
    dout = r.standard_normal((b, L, d)).astype(np.float32)
    if tag == "bf16":
        dout = synth.round_bf16(dout)
    g = dict(dout=dout)
    g["dlast"] = r.standard_normal((b, d, n)).astype(np.float32) if dlast else None
    g["h0"] = r.standard_normal((b, d, n)).astype(np.float32) if h0 else None
    return g


def gpu_backward(x, tag, g, *, D=True, z=True, bias=True, softplus=True, ckpt=None):
    from selective_state_space_38_amd import selective_scan_bwd
    dt = act_dtype(tag)
    res = selective_scan_bwd(
        to_dev(x["u"], dt), to_dev(x["delta"], dt), to_dev(x["A"], torch.float32),
        to_dev(x["B"], dt), to_dev(x["C"], dt), to_dev(g["dout"], dt),
        D=to_dev(x["D"], torch.float32) if D else None, z=to_dev(x["z"], dt) if z else None,
        delta_bias=to_dev(x["dt_bias"], torch.float32) if bias else None,
        delta_softplus=softplus, h0=to_dev(g["h0"], torch.float32),
        dlast=to_dev(g["dlast"], torch.float32), ckpt=ckpt)
    torch.cuda.synchronize()
    return {k: v.double().cpu().numpy() for k, v in res.items()}


def gpu_forward_train(x, tag, g):
    """The training-mode forward: returns (out, ckpt buffer) and checks its
    output against the plain forward's: bit for bit when no segment uses the
    look-back (whose summation path depends on timing), else to tolerance."""
    from selective_state_space_38_amd import ckpt_buffer, fwd_plan, selective_scan_fwd
    dt = act_dtype(tag)
    args = (to_dev(x["u"], dt), to_dev(x["delta"], dt), to_dev(x["A"], torch.float32),
            to_dev(x["B"], dt), to_dev(x["C"], dt))
    kw = dict(D=to_dev(x["D"], torch.float32), z=to_dev(x["z"], dt),
              delta_bias=to_dev(x["dt_bias"], torch.float32), h0=to_dev(g["h0"], torch.float32))
    ck = ckpt_buffer(args[0], x["A"].shape[1])
    out_t = selective_scan_fwd(*args, **kw, ckpt=ck)
    out_p = selective_scan_fwd(*args, **kw)
    torch.cuda.synchronize()
    b, L, d = x["u"].shape
    if fwd_plan(b, L, d, x["A"].shape[1], dt)["lookback"] == 0:
        assert torch.equal(out_t, out_p), "training-mode forward changed the output"
    else:
        a, c = out_t.double().cpu().numpy(), out_p.double().cpu().numpy()
        check("training-mode out", a, c, float(np.max(np.abs(c))), TOL[tag])
    return out_t, ck


def oracle_backward(x, g, *, D=True, z=True, bias=True, softplus=True, chans=None):
    sl = slice(None) if chans is None else chans
    return oracle.scan_bwd(
        x["u"][:, :, sl], x["delta"][:, :, sl], x["A"][sl], x["B"], x["C"],
        x["D"][sl] if D else None, x["z"][:, :, sl] if z else None,
        x["dt_bias"][sl] if bias else None, delta_softplus=softplus,
        h0=None if g["h0"] is None else g["h0"][:, sl],
        dout=g["dout"][:, :, sl], dlast=None if g["dlast"] is None else g["dlast"][:, sl])


def check_grads(got, ref, tag, keys=None):
    errs = {}
    for k in (keys or ref.keys()):
        assert k in got, f"missing gradient {k}"
        scale = float(np.max(np.abs(ref[k])))
        errs[k] = check(k, got[k], ref[k], scale, TOL[tag]) / max(scale, 1e-300)
    return errs


def test_tiny_backward_full():
    x = synth.make("tiny")
    g = _grads_in(x, "f32", 1)
    got = gpu_backward(x, "f32", g)
    ref = oracle_backward(x, g)
    errs = check_grads(got, ref, "f32")
    _log("tiny bwd " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))


BWD_SHAPES = [
    ("mamba130m", 2, 300, 100, 16),
    ("mamba2p8b", 2, 300, 100, 16),
    ("mamba130m", 1, 1, 64, 16),
    ("mamba130m", 3, 17, 1, 4),
    ("mamba130m", 1, 75, 130, 1),
    ("mamba130m", 1, 75, 130, 2),
    ("mamba130m", 1, 75, 130, 4),
    ("mamba130m", 1, 75, 130, 8),
    ("mamba130m", 1, 75, 130, 32),
    ("mamba130m", 1, 75, 70, 64),
    ("mamba2p8b", 1, 65, 70, 64),
]


@pytest.mark.parametrize("wl,b,L,d,n", BWD_SHAPES)
def test_backward_shapes(wl, b, L, d, n):
    tag = synth.WORKLOADS[wl].dtype
    x = synth.make(wl, batch=b, seqlen=L, dim=d, dstate=n, a_init="random")
    g = _grads_in(x, tag, L + d)
    _log(f"bwd {wl} b{b} L{L} d{d} n{n}")
    got = gpu_backward(x, tag, g)
    ref = oracle_backward(x, g)
    check_grads(got, ref, tag)


@pytest.mark.parametrize("drop", ["D", "z", "bias", "softplus", "h0", "dlast", "all"])
def test_backward_nullable(drop):
    x = synth.make("mamba130m", batch=2, seqlen=90, dim=70, dstate=16, a_init="random")
    kw = dict(D=True, z=True, bias=True, softplus=True)
    drops = ["D", "z", "bias", "softplus", "h0", "dlast"] if drop == "all" else [drop]
    g = _grads_in(x, "f32", 3, dlast="dlast" not in drops, h0="h0" not in drops)
    for k in drops:
        if k in kw:
            kw[k] = False
    if not kw["softplus"]:
        x["delta"] = np.abs(x["delta"]) * 0.05
        x["dt_bias"] = np.full_like(x["dt_bias"], 0.01)
    got = gpu_backward(x, "f32", g, **kw)
    ref = oracle_backward(x, g, **kw)
    assert set(got) == set(ref), (set(got), set(ref))
    check_grads(got, ref, "f32")


def test_backward_is_deterministic():
    x = synth.make("mamba2p8b", batch=2, seqlen=200, dim=192, dstate=16, a_init="random")
    g = _grads_in(x, "bf16", 4)
    a = gpu_backward(x, "bf16", g)
    b = gpu_backward(x, "bf16", g)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_backward_mid_size_full():
    """All gradients, including the channel sums dB and dC, at 1536 channels."""
    x = synth.make("mamba130m", batch=2, seqlen=512)
    g = _grads_in(x, "f32", 5)
    got = gpu_backward(x, "f32", g)
    ref = oracle_backward(x, g)
    errs = check_grads(got, ref, "f32")
    _log("130M-width bwd " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))


def test_backward_2p8b_full_size_sampled():
    """Full-size 2.8B-shaped launch.  Column-local gradients (du, ddelta, dz,
    dA, dD, ddt_bias, dh0) on sampled channels of every batch row; then dB,
    dC exactly, from a second launch whose dout and dlast are zero outside
    the sampled channels (the adjoint is then zero there, so dB and dC are
    the sums over the sampled channels alone)."""
    w = synth.WORKLOADS["mamba2p8b"]
    x = synth.make("mamba2p8b")
    g = _grads_in(x, "bf16", 6)
    r = np.random.default_rng(7)
    chans = np.unique(np.concatenate([[0, 63, 64, w.dim - 1],
                                      r.choice(w.dim, 12, replace=False)]))
    _log(f"2.8B bwd full size, channels {chans.tolist()}")
    got = gpu_backward(x, "bf16", g)
    ref = oracle_backward(x, g, chans=chans)
    cols = {"du": got["du"][:, :, chans], "ddelta": got["ddelta"][:, :, chans],
            "dz": got["dz"][:, :, chans], "dA": got["dA"][chans], "dD": got["dD"][chans],
            "ddt_bias": got["ddt_bias"][chans], "dh0": got["dh0"][:, chans]}
    check_grads(cols, ref, "bf16", keys=list(cols))
    mask = np.zeros(w.dim, bool)
    mask[chans] = True
    g2 = dict(g)
    g2["dout"] = np.where(mask, g["dout"], 0.0).astype(np.float32)
    g2["dlast"] = np.where(mask[None, :, None], g["dlast"], 0.0).astype(np.float32)
    got2 = gpu_backward(x, "bf16", g2)
    check_grads({"dB": got2["dB"], "dC": got2["dC"]}, ref, "bf16", keys=["dB", "dC"])
    assert np.all(got2["du"][:, :, ~mask] == 0.0)


def test_backward_seq1m_full_size_sampled():
    """The million-token sequence at full size (every chain split into
    look-back segments of the adjoint carry), as the 2.8B test: column-local
    gradients on two channels of different channel blocks, then dB and dC
    from a launch whose dout and dlast are zero outside those channels."""
    w = synth.WORKLOADS["seq1m"]
    x = synth.make("seq1m")
    g = _grads_in(x, "f32", 19)
    chans = np.array([0, 191])
    _log(f"million-token bwd full size, channels {chans.tolist()}")
    got = gpu_backward(x, "f32", g)
    cols = {"du": got["du"][:, :, chans], "ddelta": got["ddelta"][:, :, chans],
            "dz": got["dz"][:, :, chans], "dA": got["dA"][chans], "dD": got["dD"][chans],
            "ddt_bias": got["ddt_bias"][chans], "dh0": got["dh0"][:, chans]}
    del got
    ref = oracle_backward(x, g, chans=chans)
    check_grads(cols, ref, "f32", keys=list(cols))
    mask = np.zeros(w.dim, bool)
    mask[chans] = True
    g2 = dict(g)
    g2["dout"] = np.where(mask, g["dout"], 0.0).astype(np.float32)
    g2["dlast"] = np.where(mask[None, :, None], g["dlast"], 0.0).astype(np.float32)
    got2 = gpu_backward(x, "f32", g2)
    check_grads({"dB": got2["dB"], "dC": got2["dC"]}, ref, "f32", keys=["dB", "dC"])
    assert np.all(got2["du"][:, :, ~mask] == 0.0)


@pytest.mark.parametrize("wl,b,L,d", [
    ("tiny", 1, 64, 16),
    ("mamba130m", 2, 301, 130),
    ("mamba130m", 1, 200, 64 * 300),     # 256 whole chains + split remainder
])
def test_training_pair(wl, b, L, d):
    """selective_scan_fwd with ckpt, then selective_scan_bwd with the same
    ckpt: the backward reads the forward's checkpoints instead of running its
    own forward pass; every gradient against the oracle."""
    tag = synth.WORKLOADS[wl].dtype
    n = 4 if wl == "tiny" else 16
    x = synth.make(wl, batch=b, seqlen=L, dim=d, dstate=n, a_init="random")
    g = _grads_in(x, tag, 12)
    _, ck = gpu_forward_train(x, tag, g)
    got = gpu_backward(x, tag, g, ckpt=ck)
    if d <= 256:
        ref = oracle_backward(x, g)
        check_grads(got, ref, tag)
    else:
        chans = np.array([0, 5, 16383, 16384, 17000, d - 1])
        ref = oracle_backward(x, g, chans=chans)
        cols = {"du": got["du"][:, :, chans], "ddelta": got["ddelta"][:, :, chans],
                "dz": got["dz"][:, :, chans], "dA": got["dA"][chans], "dD": got["dD"][chans],
                "ddt_bias": got["ddt_bias"][chans], "dh0": got["dh0"][:, chans]}
        check_grads(cols, ref, tag, keys=list(cols))


def test_training_pair_2p8b_full_size():
    """The 2.8B layer: training-mode forward, then the backward from its
    checkpoints, checked on sampled channels as in the full-size test."""
    w = synth.WORKLOADS["mamba2p8b"]
    x = synth.make("mamba2p8b")
    g = _grads_in(x, "bf16", 13)
    _, ck = gpu_forward_train(x, "bf16", g)
    got = gpu_backward(x, "bf16", g, ckpt=ck)
    chans = np.array([0, 63, 64, 4095, 4096, w.dim - 1])
    ref = oracle_backward(x, g, chans=chans)
    cols = {"du": got["du"][:, :, chans], "ddelta": got["ddelta"][:, :, chans],
            "dz": got["dz"][:, :, chans], "dA": got["dA"][chans], "dD": got["dD"][chans],
            "ddt_bias": got["ddt_bias"][chans], "dh0": got["dh0"][:, chans]}
    check_grads(cols, ref, "bf16", keys=list(cols))


@pytest.mark.parametrize("split,whole,L", [(4, 1, 700), (8, 0, 515), (3, 2, 300)])
def test_training_pair_split_chains(split, whole, L):
    """Backward from checkpoints with chains split into segments that
    exchange the adjoint carry by a reverse look-back (forced here on a small
    shape: `whole` chains run whole, the rest in `split` segments); every
    gradient, including the channel sums, against the oracle."""
    x = synth.make("mamba130m", batch=2, seqlen=L, dim=130, dstate=16, a_init="random")
    g = _grads_in(x, "f32", 14)
    _, ck = gpu_forward_train(x, "f32", g)
    with env(SSM_FORCE_BWD_SPLIT=split, SSM_FORCE_BWD_WHOLE=whole):
        got = gpu_backward(x, "f32", g, ckpt=ck)
    ref = oracle_backward(x, g)
    check_grads(got, ref, "f32")


@pytest.mark.parametrize("n,tag", [(32, "f32"), (64, "f32"), (64, "bf16"), (8, "bf16")])
def test_training_pair_split_other_state_counts(n, tag):
    """The split backward with other state counts: 8 state groups (N = 32,
    64; N = 64 keeps one partial-sum buffer and a mid-chunk barrier) and two
    (N = 8), through the aggregate pass and the look-back."""
    wl = "mamba130m" if tag == "f32" else "mamba2p8b"
    x = synth.make(wl, batch=2, seqlen=300, dim=70, dstate=n, a_init="random")
    g = _grads_in(x, tag, 40 + n)
    _, ck = gpu_forward_train(x, tag, g)
    _log(f"split bwd n{n} {tag}")
    with env(SSM_FORCE_BWD_SPLIT=3, SSM_FORCE_BWD_WHOLE=1):
        got = gpu_backward(x, tag, g, ckpt=ck)
    ref = oracle_backward(x, g)
    check_grads(got, ref, tag)


def test_split_backward_without_dlast_and_h0():
    x = synth.make("mamba2p8b", batch=1, seqlen=400, dim=200, dstate=16, a_init="random")
    g = _grads_in(x, "bf16", 15, dlast=False, h0=False)
    _, ck = gpu_forward_train(x, "bf16", g)
    with env(SSM_FORCE_BWD_SPLIT=5, SSM_FORCE_BWD_WHOLE=1):
        got = gpu_backward(x, "bf16", g, ckpt=ck)
    ref = oracle_backward(x, g)
    check_grads(got, ref, "bf16")


def test_split_backward_wait_bound_reports_timeout():
    """A zero spin bound ends the adjoint-carry walk at the first unpublished
    record; the kernel still exits and the error counter reports it."""
    from selective_state_space_38_amd import check_device_errors
    x = synth.make("mamba130m", batch=1, seqlen=2048, dim=64, dstate=16, a_init="random")
    g = _grads_in(x, "f32", 16)
    _, ck = gpu_forward_train(x, "f32", g)
    check_device_errors()
    with env(SSM_FORCE_BWD_SPLIT=16, SSM_FORCE_BWD_WHOLE=0, SSM_TEST_SPIN_LIMIT=0):
        gpu_backward(x, "f32", g, ckpt=ck)
    with pytest.raises(RuntimeError, match="SSM_ETIMEOUT"):
        check_device_errors()
    with env(SSM_FORCE_BWD_SPLIT=16, SSM_FORCE_BWD_WHOLE=0):
        got = gpu_backward(x, "f32", g, ckpt=ck)
    check_device_errors()
    check_grads(got, oracle_backward(x, g), "f32")


def test_training_pair_long_sequence_all_split():
    """Few channel blocks and a long sequence (B = 1, D = 256: 4 chains): with
    checkpoints every chain is split (64 segments of 512 steps here), so the
    backward fills the GPU; every gradient on sampled channels."""
    x = synth.make("seq1m", seqlen=32768)
    g = _grads_in(x, "f32", 17)
    _, ck = gpu_forward_train(x, "f32", g)
    got = gpu_backward(x, "f32", g, ckpt=ck)
    chans = np.array([0, 63, 64, 200, 255])
    ref = oracle_backward(x, g, chans=chans)
    cols = {"du": got["du"][:, :, chans], "ddelta": got["ddelta"][:, :, chans],
            "dz": got["dz"][:, :, chans], "dA": got["dA"][chans], "dD": got["dD"][chans],
            "ddt_bias": got["ddt_bias"][chans], "dh0": got["dh0"][:, chans]}
    check_grads(cols, ref, "f32", keys=list(cols))
    # dB and dC need every channel: all 256 are cheap enough here
    ref_all = oracle_backward(x, g)
    check_grads({"dB": got["dB"], "dC": got["dC"]}, ref_all, "f32", keys=["dB", "dC"])


@pytest.mark.parametrize("split,tag", [(16, "f32"), (64, "f32"), (16, "bf16")])
def test_split_backward_stress(split, tag):
    """The reverse look-back of the adjoint carry under repetition: every
    chain split into `split` segments (128 or 32 steps at L = 2048), the
    backward run 20 times from the same checkpoints, every run's gradients
    against the oracle and against the first run's (only the look-back's
    summation order may differ), and the device error counter after each."""
    from selective_state_space_38_amd import check_device_errors
    wl = "mamba130m" if tag == "f32" else "mamba2p8b"
    x = synth.make(wl, batch=2, seqlen=2048, dim=128, dstate=16, a_init="random")
    g = _grads_in(x, tag, 60 + split)
    _, ck = gpu_forward_train(x, tag, g)
    ref = oracle_backward(x, g)
    check_device_errors()
    first = None
    _log(f"split bwd stress split={split} {tag}")
    with env(SSM_FORCE_BWD_SPLIT=split, SSM_FORCE_BWD_WHOLE=0):
        for rep in range(20):
            got = gpu_backward(x, tag, g, ckpt=ck)
            check_device_errors()   # raises if an adjoint-carry wait timed out
            check_grads(got, ref, tag)
            if first is None:
                first = got
            else:
                for k, v in got.items():
                    scale = float(np.max(np.abs(ref[k])))
                    d = float(np.max(np.abs(v - first[k])))
                    assert d <= TOL[tag] * scale, (rep, k, d, scale)
            if rep % 5 == 0:
                _log(f"  rep {rep} ok")
