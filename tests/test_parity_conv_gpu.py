"""GPU parity of the causal depthwise conv1d + SiLU (causal_conv1d_fwd /
causal_conv1d_update) against the float64 oracle (oracle.conv1d).

Tolerance: max-abs error <= tol * max |oracle output|, tol = 1e-5 for float32
(at most 4 fused multiply-adds and the SiLU's hardware exp and reciprocal
per output) and 4e-3 for bfloat16 (the output's round-to-nearest-even alone
costs up to 2^-9 of its magnitude).  Final states are copies of inputs and
must match exactly."""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import check, gpu_available, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL = {"f32": 1e-5, "bf16": 4e-3}


def _dt(tag):
    return torch.bfloat16 if tag == "bf16" else torch.float32


def _case(seed, b, L, d, k, tag, state=True, bias=True):
    r = np.random.default_rng(seed)
    x = r.standard_normal((b, L, d)).astype(np.float32)
    if tag == "bf16":
        x = synth.round_bf16(x)
    w = (r.standard_normal((d, k)) * 0.5).astype(np.float32)
    bv = r.standard_normal(d).astype(np.float32) if bias else None
    s0 = r.standard_normal((b, d, k - 1)).astype(np.float32) if state else None
    if s0 is not None and tag == "bf16":
        s0 = synth.round_bf16(s0)
    return x, w, bv, s0


def _gpu_fwd(x, w, bv, s0, tag, activation="silu"):
    from selective_state_space_38_amd import causal_conv1d_fwd
    out, st = causal_conv1d_fwd(to_dev(x, _dt(tag)), to_dev(w, torch.float32),
                                to_dev(bv, torch.float32), to_dev(s0, torch.float32),
                                activation=activation, return_final_state=True)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), st.cpu().numpy()


SHAPES = [(1, 1, 1), (2, 3, 7), (1, 129, 64), (2, 300, 100), (1, 257, 130), (3, 40, 512)]


@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("tag", ["f32", "bf16"])
@pytest.mark.parametrize("b,L,d", SHAPES)
def test_conv_forward(k, tag, b, L, d):
    x, w, bv, s0 = _case(k * 1000 + L + d, b, L, d, k, tag)
    got, st = _gpu_fwd(x, w, bv, s0, tag)
    ref, ref_st = oracle.causal_conv1d(x, w, bv, init_state=s0)
    check("conv out", got, ref, float(np.max(np.abs(ref))), TOL[tag])
    assert np.array_equal(st, ref_st.astype(np.float32))


@pytest.mark.parametrize("opt", ["no_bias", "no_state", "no_act"])
def test_conv_optional_arguments(opt):
    x, w, bv, s0 = _case(7, 2, 150, 96, 4, "f32", state=opt != "no_state", bias=opt != "no_bias")
    act = None if opt == "no_act" else "silu"
    got, st = _gpu_fwd(x, w, bv, s0, "f32", activation=act)
    ref, ref_st = oracle.causal_conv1d(x, w, bv, init_state=s0, activation=act)
    check("conv out", got, ref, float(np.max(np.abs(ref))), TOL["f32"])
    assert np.array_equal(st, ref_st.astype(np.float32))


def test_conv_split_and_decode_bitwise():
    """The state hand-off between pieces and L decode steps reproduce the
    forward bit for bit."""
    from selective_state_space_38_amd import causal_conv1d_update
    x, w, bv, s0 = _case(8, 2, 300, 136, 4, "bf16")
    full, st_full = _gpu_fwd(x, w, bv, s0, "bf16")
    a, sa = _gpu_fwd(x[:, :131], w, bv, s0, "bf16")
    b_, sb = _gpu_fwd(x[:, 131:], w, bv, sa, "bf16")
    assert np.array_equal(np.concatenate([a, b_], axis=1), full)
    assert np.array_equal(sb, st_full)
    st = to_dev(s0, torch.float32)
    wt, bt = to_dev(w, torch.float32), to_dev(bv, torch.float32)
    xt = to_dev(x, torch.bfloat16)
    outs = []
    for t in range(40):
        outs.append(causal_conv1d_update(st, xt[:, t].contiguous(), wt, bt).double().cpu().numpy())
    assert np.array_equal(np.stack(outs, axis=1), full[:, :40])
    _, st40 = _gpu_fwd(x[:, :40], w, bv, s0, "bf16")
    assert np.array_equal(st.cpu().numpy(), st40)


@pytest.mark.parametrize("k", [1, 2, 4])
@pytest.mark.parametrize("tag", ["f32", "bf16"])
def test_conv_update_against_oracle(k, tag):
    from selective_state_space_38_amd import causal_conv1d_update
    r = np.random.default_rng(9 + k)
    b, d = 5, 333
    x = r.standard_normal((b, d)).astype(np.float32)
    if tag == "bf16":
        x = synth.round_bf16(x)
    w = r.standard_normal((d, k)).astype(np.float32)
    bv = r.standard_normal(d).astype(np.float32)
    s0 = r.standard_normal((b, d, k - 1)).astype(np.float32)
    st = to_dev(s0, torch.float32)
    got = causal_conv1d_update(st, to_dev(x, _dt(tag)), to_dev(w, torch.float32),
                               to_dev(bv, torch.float32)).double().cpu().numpy()
    ref, ref_st = oracle.conv1d_update(s0, x, w, bv)
    check("update out", got, ref, float(np.max(np.abs(ref))), TOL[tag])
    assert np.array_equal(st.cpu().numpy(), ref_st.astype(np.float32))


def test_conv_2p8b_full_size_sampled():
    """The 2.8B layer's activations (4 x 8192 x 5120, bfloat16), width 4, at
    full size; the oracle recomputes 64 sampled channels (the op is per
    channel)."""
    w8 = synth.WORKLOADS["mamba2p8b"]
    xw = synth.make("mamba2p8b")
    x = xw["u"]
    r = np.random.default_rng(11)
    w = (r.standard_normal((w8.dim, 4)) * 0.5).astype(np.float32)
    bv = r.standard_normal(w8.dim).astype(np.float32)
    got, st = _gpu_fwd(x, w, bv, None, "bf16")
    chans = np.unique(np.concatenate([[0, 7, 8, w8.dim - 1], r.choice(w8.dim, 60, replace=False)]))
    ref, ref_st = oracle.causal_conv1d(x[:, :, chans], w[chans], bv[chans])
    check("conv out", got[:, :, chans], ref, float(np.max(np.abs(ref))), TOL["bf16"])
    assert np.array_equal(st[:, chans], ref_st.astype(np.float32))
