"""GPU parity of the segment carry record and the carry combination, through
the C ABI, against the float64 oracle.

A sequence scanned in pieces ("Mamba / MambaMini" Steps 2-4): each piece's
record (sum of Delta, state reached from zero) comes from
selective_scan_fwd_aggregate, selective_scan_carry_combine folds the records
into every piece's start state, and selective_scan_fwd_h0 then produces each
piece's outputs from its true start.  Together they must reproduce the
forward over the whole sequence.  Tolerances: the state against max |state|
of the oracle and sum of Delta against max |sum of Delta|, at 1e-4 for
float32 activations and 2e-2 for bfloat16 (the forward's bounds), sum of
Delta at 1e-4 in both (its arithmetic is float32 on exactly representable
inputs); outputs as the forward's parity tests (parity_util).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import (TOL, act_dtype, check, check_forward, env, gpu_available,
                         oracle_forward, sample_columns, to_dev)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

MODES = {
    "planner": dict(SSM_FORCE_LOOKBACK=None, SSM_FORCE_SEGMENT=None),
    "whole": dict(SSM_FORCE_LOOKBACK=0, SSM_FORCE_SEGMENT=None),
    "chained": dict(SSM_FORCE_LOOKBACK=0, SSM_FORCE_SEGMENT=64),
    "lookback": dict(SSM_FORCE_LOOKBACK=1, SSM_FORCE_SEGMENT=64),
}


def _log(msg):
    print(msg, flush=True)


def _wl(tag):
    return "mamba130m" if tag == "f32" else "mamba2p8b"


def _gpu_aggregate(x, tag, h0=None, bbar="delta", sl=slice(None)):
    from selective_state_space_38_amd import selective_scan_fwd_aggregate
    dt = act_dtype(tag)
    sd, st = selective_scan_fwd_aggregate(
        to_dev(x["u"][:, sl], dt), to_dev(x["delta"][:, sl], dt), to_dev(x["A"], torch.float32),
        to_dev(x["B"][:, sl], dt), delta_bias=to_dev(x["dt_bias"], torch.float32),
        h0=None if h0 is None else to_dev(h0, torch.float32), bbar=bbar)
    torch.cuda.synchronize()
    return sd, st


def _check_record(tag, sd, st, ref_sd, ref_st):
    check("sum_delta", sd.double().cpu().numpy(), ref_sd, float(np.max(np.abs(ref_sd))), 1e-4)
    check("state", st.double().cpu().numpy(), ref_st, float(np.max(np.abs(ref_st))), TOL[tag])


@pytest.mark.parametrize("with_h0", [False, True])
@pytest.mark.parametrize("bbar", ["delta", "zoh"])
@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("tag", ["f32", "bf16"])
def test_aggregate_matches_oracle(tag, mode, bbar, with_h0):
    """Record of 600 steps (a ragged last chunk) over 96 channels (a ragged
    channel block), random A, in every carry mode of the launch plan."""
    from selective_state_space_38_amd import check_device_errors
    x = synth.make(_wl(tag), batch=2, seqlen=600, dim=96, dstate=16, a_init="random")
    h0 = np.random.default_rng(7).standard_normal((2, 96, 16)).astype(np.float32) \
        if with_h0 else None
    ref_sd, ref_st = oracle.segment_aggregate(x["u"], x["delta"], x["A"], x["B"],
                                              dt_bias=x["dt_bias"], h0=h0, bbar=bbar)
    with env(**MODES[mode]):
        sd, st = _gpu_aggregate(x, tag, h0=h0, bbar=bbar)
    check_device_errors()
    _check_record(tag, sd, st, ref_sd, ref_st)


@pytest.mark.parametrize("n", [1, 2, 4, 8, 32, 64])
def test_aggregate_state_sizes(n):
    """Every instantiated d_state, split into look-back segments."""
    x = synth.make("mamba130m", batch=1, seqlen=700, dim=130, dstate=n, a_init="random")
    ref_sd, ref_st = oracle.segment_aggregate(x["u"], x["delta"], x["A"], x["B"],
                                              dt_bias=x["dt_bias"])
    with env(SSM_FORCE_LOOKBACK=1, SSM_FORCE_SEGMENT=128):
        sd, st = _gpu_aggregate(x, "f32")
    _check_record("f32", sd, st, ref_sd, ref_st)


@pytest.mark.parametrize("tag", ["f32", "bf16"])
def test_aggregate_state_is_forward_last_state(tag):
    """With whole chains the aggregate pass takes the forward's own steps in
    the same order: its state equals the forward's last_state bit for bit."""
    from selective_state_space_38_amd import selective_scan_fwd
    x = synth.make(_wl(tag), batch=2, seqlen=333, dim=128, dstate=16)
    dt = act_dtype(tag)
    with env(SSM_FORCE_LOOKBACK=0, SSM_FORCE_SEGMENT=None):
        _, st = _gpu_aggregate(x, tag)
        _, last = selective_scan_fwd(
            to_dev(x["u"], dt), to_dev(x["delta"], dt), to_dev(x["A"], torch.float32),
            to_dev(x["B"], dt), to_dev(x["C"], dt), D=to_dev(x["D"], torch.float32),
            z=to_dev(x["z"], dt), delta_bias=to_dev(x["dt_bias"], torch.float32),
            return_last_state=True)
    torch.cuda.synchronize()
    assert torch.equal(st, last)


@pytest.mark.parametrize("tag", ["f32", "bf16"])
def test_aggregate_whole_and_split_chains(tag):
    """300 chains: 256 whole chains plus 44 split into five look-back
    segments each (the plan the 2.8B-shaped layer gets), in one launch."""
    from selective_state_space_38_amd import fwd_plan
    bsz, L, dim, n = 1, 160, 64 * 300, 16
    plan = fwd_plan(bsz, L, dim, n, act_dtype(tag))
    assert plan["whole_chains"] == 256 and plan["segments"] == 5, plan
    x = synth.make(_wl(tag), batch=bsz, seqlen=L, dim=dim, dstate=n, a_init="random")
    ref_sd, ref_st = oracle.segment_aggregate(x["u"], x["delta"], x["A"], x["B"],
                                              dt_bias=x["dt_bias"])
    sd, st = _gpu_aggregate(x, tag)
    _check_record(tag, sd, st, ref_sd, ref_st)


def test_carry_combine_matches_oracle():
    """Five records folded from a given start state; and from zeros."""
    from selective_state_space_38_amd import selective_scan_carry_combine
    r = np.random.default_rng(11)
    S, b, d, n = 5, 2, 70, 16
    sdl = r.uniform(0.0, 3.0, (S, b, d)).astype(np.float32)
    agg = r.standard_normal((S, b, d, n)).astype(np.float32)
    A = (-np.exp(r.standard_normal((d, n)))).astype(np.float32)
    h0 = r.standard_normal((b, d, n)).astype(np.float32)
    for start in (h0, None):
        ref_in, ref_out = oracle.carry_combine(sdl, agg, A, h0=start)
        h_in, h_out = selective_scan_carry_combine(
            to_dev(sdl, torch.float32), to_dev(agg, torch.float32), to_dev(A, torch.float32),
            h0=None if start is None else to_dev(start, torch.float32))
        torch.cuda.synchronize()
        scale = float(np.max(np.abs(ref_in)))
        check("h_in", h_in.double().cpu().numpy(), ref_in, scale, 1e-5)
        check("h_out", h_out.double().cpu().numpy(), ref_out, scale, 1e-5)


def _pieces_forward(x, tag, bounds, h0, bbar="delta", keep=False):
    """The sequence in pieces: every piece's record from zero, the fold from
    h0, then every piece's outputs from its start state (with `keep`, from
    the carries each piece's record call kept).  Returns the concatenated
    outputs and the state after the last piece."""
    from selective_state_space_38_amd import (record_buffer, selective_scan_carry_combine,
                                              selective_scan_fwd, selective_scan_fwd_aggregate)
    dt = act_dtype(tag)
    A = to_dev(x["A"], torch.float32)
    bias = to_dev(x["dt_bias"], torch.float32)
    Dv = to_dev(x["D"], torch.float32)
    pieces = [slice(lo, hi) for lo, hi in zip(bounds[:-1], bounds[1:])]
    dev = {k: [to_dev(x[k][:, sl], dt) for sl in pieces] for k in ("u", "delta", "z", "B", "C")}
    bufs = [record_buffer(dev["u"][i], x["A"].shape[1]) if keep else None
            for i in range(len(pieces))]
    recs = [selective_scan_fwd_aggregate(dev["u"][i], dev["delta"][i], A, dev["B"][i],
                                         delta_bias=bias, bbar=bbar, rec=bufs[i])
            for i in range(len(pieces))]
    h_in, h_out = selective_scan_carry_combine(
        torch.stack([r[0] for r in recs]), torch.stack([r[1] for r in recs]), A,
        h0=None if h0 is None else to_dev(h0, torch.float32))
    outs = [selective_scan_fwd(dev["u"][i], dev["delta"][i], A, dev["B"][i], dev["C"][i], D=Dv,
                               z=dev["z"][i], delta_bias=bias, h0=h_in[i].contiguous(),
                               bbar=bbar, rec=bufs[i])
            for i in range(len(pieces))]
    torch.cuda.synchronize()
    return torch.cat(outs, dim=1), h_out


@pytest.mark.parametrize("keep", [False, True])
@pytest.mark.parametrize("bbar", ["delta", "zoh"])
@pytest.mark.parametrize("tag", ["f32", "bf16"])
def test_sequence_in_pieces_equals_whole_forward(tag, bbar, keep):
    """Four pieces of unequal length (each long enough to be split into
    look-back segments inside its own calls) reproduce the forward over the
    whole 4,100-step sequence from a given h0."""
    bsz, L, dim, n = 1, 4100, 256, 16
    x = synth.make(_wl(tag), batch=bsz, seqlen=L, dim=dim, dstate=n, a_init="random")
    h0 = np.random.default_rng(5).standard_normal((bsz, dim, n)).astype(np.float32)
    bounds = [0, 1000, 2104, 3100, L]
    ref, ref_st = oracle_forward(x, h0=h0, bbar=bbar)
    out, st = _pieces_forward(x, tag, bounds, h0, bbar=bbar, keep=keep)
    check_forward(x, tag, out.float().cpu().numpy(), st.cpu().numpy(), ref, ref_st)


@pytest.mark.parametrize("keep", [False, True])
def test_million_token_sequence_in_eight_pieces(keep):
    """The million-token sequence as eight pieces of 131,072 steps (one
    device's share each under sequence sharding): every piece's record,
    their fold and every piece's outputs, against the oracle over the whole
    sequence on sampled columns; and the record of the whole sequence in one
    call against the oracle's."""
    from selective_state_space_38_amd import check_device_errors
    w = synth.WORKLOADS["seq1m"]
    x = synth.make(w)
    cols = sample_columns(w.batch, w.dim, 6, seed=w.seed + 7)
    _log(f"seq1m pieces: oracle on {len(cols)} columns")
    ref, ref_st = oracle_forward(x, cols=cols)
    bounds = [k * (w.seqlen // 8) for k in range(9)]
    out, st = _pieces_forward(x, "f32", bounds, None, keep=keep)
    check_device_errors()
    bb = torch.tensor([b for b, _ in cols], device="cuda")
    dd = torch.tensor([d for _, d in cols], device="cuda")
    scale = float(np.max(np.abs(ref)))
    check("out", out[bb, :, dd].double().cpu().numpy(), ref, scale, TOL["f32"])
    check("last_state", st[bb, dd].double().cpu().numpy(), ref_st, scale, TOL["f32"])
    del out
    _log("seq1m pieces ok; whole-sequence record")
    sd, agg = _gpu_aggregate(x, "f32")
    check_device_errors()
    ds = [d for _, d in cols]
    ref_sd, ref_agg = oracle.segment_aggregate(x["u"][:, :, ds], x["delta"][:, :, ds], x["A"][ds],
                                               x["B"], dt_bias=x["dt_bias"][ds])
    _check_record("f32", sd[bb, dd][None], agg[bb, dd][None], ref_sd, ref_agg)


@pytest.mark.parametrize("mode", ["lookback", "chained"])
def test_aggregate_without_softplus_or_bias(mode):
    """Delta = dt as given (softplus off, no bias), including steps large
    enough that exp(Delta A) underflows to 0 and the state resets onto the
    current input ("Mamba / MambaMini" Q&A on how Delta acts on A)."""
    from selective_state_space_38_amd import selective_scan_fwd_aggregate
    x = synth.make("mamba130m", batch=1, seqlen=400, dim=80, dstate=16, a_init="random")
    x["A"] = np.minimum(x["A"], np.float32(-0.1))
    dt = np.abs(x["delta"]) * np.float32(0.05)
    dt[:, 300:303] = np.float32(1e4)
    ref_sd, ref_st = oracle.segment_aggregate(x["u"], dt, x["A"], x["B"], delta_softplus=False)
    with env(**MODES[mode]):
        sd, st = selective_scan_fwd_aggregate(
            to_dev(x["u"], torch.float32), to_dev(dt, torch.float32),
            to_dev(x["A"], torch.float32), to_dev(x["B"], torch.float32), delta_softplus=False)
        torch.cuda.synchronize()
    _check_record("f32", sd, st, ref_sd, ref_st)


@pytest.mark.parametrize("bbar", ["delta", "zoh"])
@pytest.mark.parametrize("mode", ["planner", "lookback", "chained", "whole"])
@pytest.mark.parametrize("tag", ["f32", "bf16"])
def test_forward_from_kept_record(tag, mode, bbar):
    """A record call that keeps its inner carries, then the forward from
    them and an h0: outputs and final state against the oracle's forward
    from h0, in every carry mode of the launch plan."""
    from selective_state_space_38_amd import record_buffer, selective_scan_fwd
    x = synth.make(_wl(tag), batch=2, seqlen=600, dim=96, dstate=16, a_init="random")
    h0 = np.random.default_rng(9).standard_normal((2, 96, 16)).astype(np.float32)
    dt = act_dtype(tag)
    ref, ref_st = oracle_forward(x, h0=h0, bbar=bbar)
    ref_sd, ref_agg = oracle.segment_aggregate(x["u"], x["delta"], x["A"], x["B"],
                                               dt_bias=x["dt_bias"], bbar=bbar)
    with env(**MODES[mode]):
        u = to_dev(x["u"], dt)
        rec = record_buffer(u, 16)
        from selective_state_space_38_amd import selective_scan_fwd_aggregate
        sd, agg = selective_scan_fwd_aggregate(
            u, to_dev(x["delta"], dt), to_dev(x["A"], torch.float32), to_dev(x["B"], dt),
            delta_bias=to_dev(x["dt_bias"], torch.float32), bbar=bbar, rec=rec)
        out, st = selective_scan_fwd(
            u, to_dev(x["delta"], dt), to_dev(x["A"], torch.float32), to_dev(x["B"], dt),
            to_dev(x["C"], dt), D=to_dev(x["D"], torch.float32), z=to_dev(x["z"], dt),
            delta_bias=to_dev(x["dt_bias"], torch.float32), h0=to_dev(h0, torch.float32),
            return_last_state=True, bbar=bbar, rec=rec)
        torch.cuda.synchronize()
    _check_record(tag, sd, agg, ref_sd, ref_agg)
    check_forward(x, tag, out.float().cpu().numpy(), st.cpu().numpy(), ref, ref_st)


def test_forward_from_kept_record_whole_and_split_chains():
    """The 2.8B-style plan (256 whole chains, 44 split into five segments)
    from a kept record: whole chains start from h0, split segments from their
    kept carries."""
    from selective_state_space_38_amd import (record_buffer, selective_scan_fwd,
                                              selective_scan_fwd_aggregate)
    bsz, L, dim, n = 1, 160, 64 * 300, 16
    x = synth.make("mamba2p8b", batch=bsz, seqlen=L, dim=dim, dstate=n, a_init="random")
    h0 = np.random.default_rng(10).standard_normal((bsz, dim, n)).astype(np.float32)
    ref, ref_st = oracle_forward(x, h0=h0)
    dt = torch.bfloat16
    u = to_dev(x["u"], dt)
    rec = record_buffer(u, n)
    selective_scan_fwd_aggregate(u, to_dev(x["delta"], dt), to_dev(x["A"], torch.float32),
                                 to_dev(x["B"], dt), delta_bias=to_dev(x["dt_bias"], torch.float32),
                                 rec=rec)
    out, st = selective_scan_fwd(
        u, to_dev(x["delta"], dt), to_dev(x["A"], torch.float32), to_dev(x["B"], dt),
        to_dev(x["C"], dt), D=to_dev(x["D"], torch.float32), z=to_dev(x["z"], dt),
        delta_bias=to_dev(x["dt_bias"], torch.float32), h0=to_dev(h0, torch.float32),
        return_last_state=True, rec=rec)
    torch.cuda.synchronize()
    check_forward(x, "bf16", out.float().cpu().numpy(), st.cpu().numpy(), ref, ref_st)
