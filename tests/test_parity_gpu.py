"""GPU parity: the HIP path through the C ABI against the float64 oracle on the
same seeded inputs (tolerances in parity_util)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import (TOL, check, check_forward, env, gpu_available, gpu_forward,
                         oracle_forward, sample_columns, to_dev, act_dtype)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _case(name, **kw):
    return synth.make(name, **kw)


def _log(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- forward --

def test_tiny_workload_full():
    x = _case("tiny")
    got, st = gpu_forward(x, "f32")
    ref, ref_st = oracle_forward(x)
    e1, e2, s = check_forward(x, "f32", got, st, ref, ref_st)
    _log(f"tiny: err {e1:.2e} state {e2:.2e} scale {s:.2f}")


RAGGED = [
    # (workload for distributions, batch, L, dim, N, a_init)
    ("mamba130m", 2, 300, 100, 16, "s4d"),
    ("mamba2p8b", 2, 300, 100, 16, "random"),
    ("mamba130m", 1, 1, 64, 16, "random"),
    ("mamba130m", 3, 17, 1, 4, "random"),
    ("mamba130m", 1, 257, 130, 1, "random"),
    ("mamba130m", 1, 257, 130, 2, "random"),
    ("mamba130m", 1, 257, 130, 4, "random"),
    ("mamba130m", 1, 257, 130, 8, "random"),
    ("mamba130m", 1, 257, 130, 32, "random"),
    ("mamba130m", 1, 257, 130, 64, "random"),
    ("mamba2p8b", 1, 129, 70, 64, "random"),
    # bfloat16 with eight helper waves: 32 states (eight scan waves, 1024-thread
    # workgroups) and an odd channel count (helper runs of two channels take
    # the element path)
    ("mamba2p8b", 2, 300, 100, 32, "random"),
    ("mamba2p8b", 1, 129, 131, 16, "random"),
    ("mamba130m", 1, 129, 131, 16, "random"),
]


@pytest.mark.parametrize("wl,b,L,d,n,a_init", RAGGED)
def test_ragged_shapes(wl, b, L, d, n, a_init):
    tag = synth.WORKLOADS[wl].dtype
    x = _case(wl, batch=b, seqlen=L, dim=d, dstate=n, a_init=a_init)
    _log(f"ragged {wl} b{b} L{L} d{d} n{n} {a_init}")
    got, st = gpu_forward(x, tag)
    ref, ref_st = oracle_forward(x)
    check_forward(x, tag, got, st, ref, ref_st)


@pytest.mark.parametrize("tag", ["f32", "bf16"])
@pytest.mark.parametrize("drop", ["D", "z", "bias", "softplus", "last", "all"])
def test_nullable_arguments(tag, drop):
    wl = "mamba130m" if tag == "f32" else "mamba2p8b"
    x = _case(wl, batch=2, seqlen=200, dim=80, dstate=16, a_init="random")
    kw = dict(D=True, z=True, bias=True, softplus=True, last=True)
    if drop == "all":
        kw.update(D=False, z=False, bias=False, last=False)
    else:
        kw[drop] = False
    if not kw["softplus"]:
        # without softplus Delta = dt + dt_bias must be kept positive by the
        # inputs themselves
        x["delta"] = np.abs(x["delta"]) * 0.05
        if tag == "bf16":
            x["delta"] = synth.round_bf16(x["delta"])
        x["dt_bias"] = np.full_like(x["dt_bias"], 0.01)
    _log(f"nullable {tag} drop={drop}")
    got, st = gpu_forward(x, tag, **kw)
    okw = {k: v for k, v in kw.items() if k != "last"}
    ref, ref_st = oracle_forward(x, **okw)
    check_forward(x, tag, got, st, ref, ref_st)


@pytest.mark.parametrize("tag", ["f32", "bf16"])
@pytest.mark.parametrize("lookback,seg", [(0, 32), (1, 32), (1, 256), (0, 16), (1, 16)])
def test_segment_carry_modes(tag, lookback, seg):
    """Many short segments exercise the chained hand-off and the decoupled
    look-back (aggregates, walks over several predecessors)."""
    from selective_state_space_38_amd import fwd_plan
    wl = "mamba130m" if tag == "f32" else "mamba2p8b"
    x = _case(wl, batch=2, seqlen=1000, dim=96, dstate=16, a_init="random")
    _log(f"modes {tag} lookback={lookback} seg={seg}")
    with env(SSM_FORCE_LOOKBACK=lookback, SSM_FORCE_SEGMENT=seg):
        plan = fwd_plan(2, 1000, 96, 16, act_dtype(tag))
        assert plan["segment_len"] == seg and plan["lookback"] == lookback, plan
        got, st = gpu_forward(x, tag)
    ref, ref_st = oracle_forward(x)
    check_forward(x, tag, got, st, ref, ref_st)


@pytest.mark.parametrize("tag", ["f32", "bf16"])
@pytest.mark.parametrize("lookback,seg,first", [(1, 96, 32), (1, 96, 160), (0, 64, 16),
                                                (1, 16, 48)])
def test_first_segment_length(tag, lookback, seg, first):
    """A first segment shorter or longer than the others: every segment's
    bounds and carry records follow from the two lengths."""
    from selective_state_space_38_amd import fwd_plan
    wl = "mamba130m" if tag == "f32" else "mamba2p8b"
    L = 1000
    x = _case(wl, batch=2, seqlen=L, dim=96, dstate=16, a_init="random")
    _log(f"first segment {tag} lookback={lookback} seg={seg} first={first}")
    with env(SSM_FORCE_LOOKBACK=lookback, SSM_FORCE_SEGMENT=seg, SSM_FORCE_FIRST_SEGMENT=first):
        plan = fwd_plan(2, L, 96, 16, act_dtype(tag))
        s_ = plan["segment_len"]
        assert plan["first_segment_len"] == first and plan["segments"] > 2, plan
        assert first + (plan["segments"] - 2) * s_ < L <= first + (plan["segments"] - 1) * s_
        got, st = gpu_forward(x, tag)
    ref, ref_st = oracle_forward(x)
    check_forward(x, tag, got, st, ref, ref_st)


@pytest.mark.parametrize("tag", ["f32", "bf16"])
@pytest.mark.parametrize("groups_per", [1, 2, 4, 8])
def test_state_group_layouts(groups_per, tag):
    """Every instantiated split of 16 states over waves gives the same answer."""
    wl = "mamba130m" if tag == "f32" else "mamba2p8b"
    x = _case(wl, batch=2, seqlen=190, dim=70, dstate=16, a_init="random")
    with env(SSM_FORCE_STATES_PER_GROUP=16 // groups_per):
        got, st = gpu_forward(x, tag)
    ref, ref_st = oracle_forward(x)
    check_forward(x, tag, got, st, ref, ref_st)


def test_initial_state_and_resume():
    """h0 is honoured, and splitting the sequence with h0 = last_state of the
    first part reproduces the whole ("Mamba / MambaMini" Step 4)."""
    x = _case("mamba130m", batch=2, seqlen=500, dim=72, dstate=16, a_init="random")
    h0 = np.random.default_rng(5).standard_normal((2, 72, 16)).astype(np.float32)
    got, st = gpu_forward(x, "f32", h0=h0)
    ref, ref_st = oracle_forward(x, h0=h0)
    check_forward(x, "f32", got, st, ref, ref_st)
    # resume from the GPU's own state
    L1 = 203
    head = dict(x, u=x["u"][:, :L1], delta=x["delta"][:, :L1], z=x["z"][:, :L1],
                B=x["B"][:, :L1], C=x["C"][:, :L1])
    tail = dict(x, u=x["u"][:, L1:], delta=x["delta"][:, L1:], z=x["z"][:, L1:],
                B=x["B"][:, L1:], C=x["C"][:, L1:])
    o1, s1 = gpu_forward(head, "f32", h0=h0)
    o2, s2 = gpu_forward(tail, "f32", h0=s1)
    check_forward(x, "f32", np.concatenate([o1, o2], axis=1), s2, ref, ref_st)


def test_zero_delta_keeps_state_bitwise():
    """softplus off, dt = bias = 0 -> Abar = 1, Bbar = 0: the final state is
    the initial state bit for bit (reading guide FAQ on small Delta)."""
    x = _case("mamba130m", batch=2, seqlen=300, dim=64, dstate=16, a_init="random")
    x["delta"] = np.zeros_like(x["delta"])
    x["dt_bias"] = np.zeros_like(x["dt_bias"])
    h0 = np.random.default_rng(6).standard_normal((2, 64, 16)).astype(np.float32)
    for lookback, seg in ((0, 0), (1, 64), (0, 64)):
        with env(SSM_FORCE_LOOKBACK=lookback if seg else None,
                 SSM_FORCE_SEGMENT=seg or None):
            _, st = gpu_forward(x, "f32", softplus=False, h0=h0)
        assert np.array_equal(st, h0), (lookback, seg)


def test_column_independence_bitwise():
    """Perturbing one channel and one batch row leaves every other column's
    outputs and final state bit-identical ("Mamba / MambaMini" Q&A:
    elementwise)."""
    x = _case("mamba130m", batch=3, seqlen=257, dim=130, dstate=16, a_init="random")
    o1, s1 = gpu_forward(x, "f32")
    y = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in x.items()}
    y["u"][:, :, 77] += 1.0
    y["delta"][1] -= 0.5
    o2, s2 = gpu_forward(y, "f32")
    keep = np.ones(o1.shape, bool)
    keep[:, :, 77] = False
    keep[1] = False
    assert np.array_equal(o1[keep], o2[keep])
    ks = np.ones(s1.shape, bool)
    ks[:, 77] = False
    ks[1] = False
    assert np.array_equal(s1[ks], s2[ks])


def test_chained_mode_is_deterministic():
    x = _case("mamba2p8b", batch=2, seqlen=2100, dim=192, dstate=16, a_init="random")
    with env(SSM_FORCE_LOOKBACK=0, SSM_FORCE_SEGMENT=256):
        a, sa = gpu_forward(x, "bf16")
        b, sb = gpu_forward(x, "bf16")
    assert np.array_equal(a, b) and np.array_equal(sa, sb)


def test_carry_wait_bound_reports_timeout():
    """A zero spin bound makes every wait that is not satisfied at once give
    up; the kernel still exits and the device error counter reports it."""
    from selective_state_space_38_amd import check_device_errors
    x = _case("mamba130m", batch=1, seqlen=4096, dim=64, dstate=16, a_init="random")
    check_device_errors()  # clear
    with env(SSM_FORCE_LOOKBACK=0, SSM_FORCE_SEGMENT=16, SSM_TEST_SPIN_LIMIT=0):
        gpu_forward(x, "f32")
    with pytest.raises(RuntimeError, match="SSM_ETIMEOUT"):
        check_device_errors()
    gpu_forward(x, "f32")
    check_device_errors()  # a normal call leaves the counter at zero


@pytest.mark.parametrize("split", [None, 2, 8])
def test_whole_and_split_chains(split):
    """More chains than CUs: 256 chains run whole and the rest are split into
    look-back segments (the planner's choice, or a forced split count; with a
    forced split of 8 the first segment is also given its own length)."""
    from selective_state_space_38_amd import fwd_plan
    x = _case("mamba130m", batch=1, seqlen=600, dim=64 * 300, dstate=16, a_init="random")
    first = 96 if split == 8 else 0
    with env(SSM_FORCE_SPLIT=split, SSM_FORCE_FIRST_SEGMENT=first):
        plan = fwd_plan(1, 600, 64 * 300, 16)
        got, st = gpu_forward(x, "f32")
    assert plan["whole_chains"] == 256 and plan["segments"] > 1, plan
    assert plan["first_segment_len"] == (first or plan["segment_len"]), plan
    _log(f"mixed plan {plan}")
    # columns of whole chains, of split chains and the block edges
    cols = [(0, d) for d in (0, 63, 64, 16383, 16384, 16385, 17000, 19199)]
    ref, ref_st = oracle_forward(x, cols=cols)
    g_out = np.stack([got[b, :, d] for b, d in cols])
    g_st = np.stack([st[b, d] for b, d in cols])
    scale = float(np.max(np.abs(ref)))
    check("out", g_out, ref, scale, TOL["f32"])
    check("last_state", g_st, ref_st, scale, TOL["f32"])


def test_lookback_wait_bound_reports_timeout():
    """The same for the windowed look-back walk: predecessors not yet
    published at the first poll end the walk, the kernel exits and the error
    counter reports it."""
    from selective_state_space_38_amd import check_device_errors
    x = _case("mamba130m", batch=1, seqlen=4096, dim=64, dstate=16, a_init="random")
    check_device_errors()  # clear
    with env(SSM_FORCE_LOOKBACK=1, SSM_FORCE_SEGMENT=16, SSM_TEST_SPIN_LIMIT=0):
        gpu_forward(x, "f32")
    with pytest.raises(RuntimeError, match="SSM_ETIMEOUT"):
        check_device_errors()
    with env(SSM_FORCE_LOOKBACK=1, SSM_FORCE_SEGMENT=16):
        got, st = gpu_forward(x, "f32")
    check_device_errors()
    ref, ref_st = oracle_forward(x)
    check_forward(x, "f32", got, st, ref, ref_st)


# ------------------------------------------------------- full-size workloads --

def test_workload_mamba130m_full():
    x = _case("mamba130m")
    _log("130M full-size")
    got, st = gpu_forward(x, "f32")
    ref, ref_st = oracle_forward(x)
    e1, e2, s = check_forward(x, "f32", got, st, ref, ref_st)
    _log(f"130M: err/scale {e1 / s:.2e} state err/scale {e2 / s:.2e}")


@pytest.mark.parametrize("name,count", [("mamba2p8b", 48), ("seq1m", 6)])
def test_workload_sampled_columns(name, count):
    """Full-size launch as the benchmark runs it; the oracle recomputes a
    sample of whole (batch, channel) columns."""
    w = synth.WORKLOADS[name]
    x = _case(name)
    _log(f"{name} full-size, {count} sampled columns")
    got, st = gpu_forward(x, w.dtype)
    cols = sample_columns(w.batch, w.dim, count, seed=w.seed)
    ref, ref_st = oracle_forward(x, cols=cols)
    g_out = np.stack([got[b, :, d] for b, d in cols])
    g_st = np.stack([st[b, d] for b, d in cols])
    scale = float(np.max(np.abs(ref)))
    e1 = check("out", g_out, ref, scale, TOL[w.dtype])
    e2 = check("last_state", g_st, ref_st, scale, TOL[w.dtype])
    _log(f"{name}: err/scale {e1 / scale:.2e} state {e2 / scale:.2e}")
    assert np.all(np.isfinite(got))


# ------------------------------------------------------------------ decode --

def _gpu_update(x, tag, state, *, D=True, z=True, bias=True, softplus=True):
    from selective_state_space_38_amd import selective_state_update
    dt = act_dtype(tag)
    st = to_dev(state, torch.float32)
    out = selective_state_update(
        st, to_dev(x["u"], dt), to_dev(x["delta"], dt), to_dev(x["A"], torch.float32),
        to_dev(x["B"], dt), to_dev(x["C"], dt),
        D=to_dev(x["D"], torch.float32) if D else None, z=to_dev(x["z"], dt) if z else None,
        dt_bias=to_dev(x["dt_bias"], torch.float32) if bias else None, dt_softplus=softplus)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), st.cpu().numpy()


def _check_update(x, tag, got, gst, **kw):
    ref, ref_st = oracle.state_update(
        x["state"], x["u"], x["delta"], x["A"], x["B"], x["C"],
        x["D"] if kw.get("D", True) else None, x["z"] if kw.get("z", True) else None,
        x["dt_bias"] if kw.get("bias", True) else None, kw.get("softplus", True))
    scale = float(np.max(np.abs(ref)))
    check("decode out", got, ref, scale, TOL[tag])
    check("decode state", gst, ref_st, scale, TOL[tag])


def test_decode_workload_full():
    x = _case("decode")
    got, gst = _gpu_update(x, "bf16", x["state"])
    _check_update(x, "bf16", got, gst)


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("tag", ["f32", "bf16"])
def test_decode_shapes(n, tag):
    import dataclasses
    w = dataclasses.replace(synth.WORKLOADS["decode"], dtype=tag)
    x = synth.make(w, batch=3, dim=77, dstate=n, a_init="random")
    got, gst = _gpu_update(x, tag, x["state"])
    _check_update(x, tag, got, gst)


@pytest.mark.parametrize("drop", ["D", "z", "bias", "softplus"])
def test_decode_nullable(drop):
    x = synth.make("decode", batch=4, dim=300, a_init="random")
    kw = dict(D=True, z=True, bias=True, softplus=True)
    kw[drop] = False
    if drop == "softplus":
        # without softplus the inputs themselves keep Delta positive
        x["delta"] = synth.round_bf16(np.abs(x["delta"]) * 0.05)
        x["dt_bias"] = np.full_like(x["dt_bias"], 0.01)
    got, gst = _gpu_update(x, "bf16", x["state"], **kw)
    _check_update(x, "bf16", got, gst, **kw)


def test_decode_zero_delta_keeps_state_bitwise():
    x = synth.make("decode", batch=2, dim=128, a_init="random")
    x["delta"] = np.zeros_like(x["delta"])
    x["dt_bias"] = np.zeros_like(x["dt_bias"])
    _, gst = _gpu_update(x, "bf16", x["state"], softplus=False)
    assert np.array_equal(gst, x["state"])


@pytest.mark.parametrize("tag", ["f32", "bf16"])
def test_decode_loop_equals_forward(tag):
    """L single-token updates from h0 reproduce the forward's outputs and final
    state (reading guide FAQ: recurrent decoding)."""
    wl = "mamba130m" if tag == "f32" else "mamba2p8b"
    x = _case(wl, batch=2, seqlen=40, dim=96, dstate=16, a_init="random")
    h0 = np.random.default_rng(7).standard_normal((2, 96, 16)).astype(np.float32)
    fo, fst = gpu_forward(x, tag, h0=h0)
    st = h0.copy()
    outs = []
    for t in range(40):
        step = dict(u=x["u"][:, t], delta=x["delta"][:, t], z=x["z"][:, t],
                    B=x["B"][:, t], C=x["C"][:, t], A=x["A"], D=x["D"],
                    dt_bias=x["dt_bias"])
        o, st = _gpu_update(step, tag, st)
        outs.append(o)
    outs = np.stack(outs, axis=1)
    ref, ref_st = oracle_forward(x, h0=h0)
    scale = float(np.max(np.abs(ref)))
    check("loop vs forward out", outs, fo.astype(np.float64), scale, TOL[tag])
    check("loop vs forward state", st, fst.astype(np.float64), scale, TOL[tag])
    check("loop vs oracle", outs, ref, scale, TOL[tag])
