"""HIP graph capture of the decode step, of the allocation-free forward and of
a kept-carry record with the forward from it.

The binding launches on the current stream, so torch.cuda.graph captures the
library's kernels.  Each graph is replayed several times with eager work and
synchronisations between the replays, and every replay is checked against
the same calls run eagerly: the decode bit for bit (same kernels, same
inputs), the forward, whose look-back may combine carries in another order,
to the parity tolerance.  Neither path records a memset: the forward clears
its carry words with a fill kernel."""

import numpy as np
import pytest
import torch

import synth
from parity_util import TOL, check, gpu_available, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _bf16(r, shape):
    return synth.round_bf16(r.standard_normal(shape).astype(np.float32))


def test_decode_steps_replayed_from_a_graph():
    from selective_state_space_38_amd import check_device_errors, selective_state_update
    dev = torch.device("cuda", 0)
    x = synth.make("decode")                         # 256 x 5120, d_state 16, bf16
    b, d = x["u"].shape
    n = x["A"].shape[1]
    r = np.random.default_rng(11)
    steps = 4
    act = torch.bfloat16
    ins = [dict(x=to_dev(_bf16(r, (b, d)), act), dt=to_dev(_bf16(r, (b, d)), act),
                z=to_dev(_bf16(r, (b, d)), act), B=to_dev(_bf16(r, (b, n)), act),
                C=to_dev(_bf16(r, (b, n)), act)) for _ in range(steps)]
    A, D = to_dev(x["A"], torch.float32), to_dev(x["D"], torch.float32)
    bias = to_dev(x["dt_bias"], torch.float32)
    state0 = to_dev(x["state"], torch.float32)

    def run(state, outs):
        for k in range(steps):
            v = ins[k]
            selective_state_update(state, v["x"], v["dt"], A, v["B"], v["C"], D=D, z=v["z"],
                                   dt_bias=bias, dt_softplus=True, out=outs[k])

    state_e = state0.clone()
    outs_e = [torch.empty((b, d), dtype=act, device=dev) for _ in range(steps)]
    run(state_e, outs_e)
    torch.cuda.synchronize()

    state_g = state0.clone()
    outs_g = [torch.empty((b, d), dtype=act, device=dev) for _ in range(steps)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                    # warm-up before capture
        run(state0.clone(), [torch.empty_like(o) for o in outs_g])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(state_g, outs_g)

    other = state0.clone()
    for rep in range(3):
        state_g.copy_(state0)
        for o in outs_g:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in range(steps):
            assert torch.equal(outs_g[k], outs_e[k]), (rep, k)
        assert torch.equal(state_g, state_e), rep
        # eager work between replays: more decode steps on another state
        run(other, [torch.empty_like(o) for o in outs_g])
        torch.cuda.synchronize()
    check_device_errors(dev)


def test_noalloc_forward_replayed_from_a_graph():
    from selective_state_space_38_amd import (check_device_errors, fwd_plan,
                                              selective_scan_fwd)
    dev = torch.device("cuda", 0)
    # 4 chains of 65,536 steps: every chain split into look-back segments, so
    # the graph holds the carry words' fill kernel and the segment hand-off
    x = synth.make("seq1m", seqlen=65536)
    bsz, L, dim = x["u"].shape
    n = x["A"].shape[1]
    plan = fwd_plan(bsz, L, dim, n, torch.float32)
    assert plan["segments"] > 2 and plan["lookback"] == 1, plan
    f32 = torch.float32
    t = {k: to_dev(x[k], f32) for k in ("u", "delta", "A", "B", "C", "D", "z", "dt_bias")}

    def fwd(out, last):
        selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                           delta_bias=t["dt_bias"], delta_softplus=True, out=out,
                           last_state=last, return_last_state=True, no_alloc=True)

    out_e = torch.empty_like(t["u"])
    last_e = torch.empty((bsz, dim, n), dtype=f32, device=dev)
    fwd(out_e, last_e)                               # also looks up the static array
    torch.cuda.synchronize()

    out_g, last_g = torch.empty_like(out_e), torch.empty_like(last_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd(torch.empty_like(out_e), torch.empty_like(last_e))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(out_g, last_g)

    ref_out = out_e.double().cpu().numpy()
    ref_last = last_e.double().cpu().numpy()
    scale = float(np.max(np.abs(ref_out)))
    scratch_out, scratch_last = torch.empty_like(out_e), torch.empty_like(last_e)
    for rep in range(3):
        out_g.zero_()
        last_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        check(f"graph out (replay {rep})", out_g.double().cpu().numpy(), ref_out, scale,
              TOL["f32"])
        check(f"graph last_state (replay {rep})", last_g.double().cpu().numpy(), ref_last,
              scale, TOL["f32"])
        # eager work between replays: the same entry point on the same array
        fwd(scratch_out, scratch_last)
        torch.cuda.synchronize()
    check_device_errors(dev)


def test_kept_record_and_forward_replayed_from_a_graph():
    """A piece's record keeping its inner carries, then the piece's forward
    from them and an h0, captured together: both take their scratch from the
    caller's record buffer, so neither allocates, and the record clears its
    carry words with a fill kernel."""
    from selective_state_space_38_amd import (check_device_errors, fwd_plan, record_buffer,
                                              selective_scan_fwd, selective_scan_fwd_aggregate)
    dev = torch.device("cuda", 0)
    x = synth.make("seq1m", seqlen=65536)
    bsz, L, dim = x["u"].shape
    n = x["A"].shape[1]
    plan = fwd_plan(bsz, L, dim, n, torch.float32)
    assert plan["segments"] > 2 and plan["lookback"] == 1, plan
    f32 = torch.float32
    t = {k: to_dev(x[k], f32) for k in ("u", "delta", "A", "B", "C", "D", "z", "dt_bias")}
    h0 = to_dev(np.random.default_rng(12).standard_normal((bsz, dim, n)).astype(np.float32), f32)

    def run(rec, sd, agg, out, last):
        selective_scan_fwd_aggregate(t["u"], t["delta"], t["A"], t["B"], delta_bias=t["dt_bias"],
                                     sum_delta=sd, state=agg, rec=rec)
        selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                           delta_bias=t["dt_bias"], h0=h0, out=out, last_state=last,
                           return_last_state=True, rec=rec)

    def bufs():
        return (record_buffer(t["u"], n), torch.empty((bsz, dim), dtype=f32, device=dev),
                torch.empty((bsz, dim, n), dtype=f32, device=dev), torch.empty_like(t["u"]),
                torch.empty((bsz, dim, n), dtype=f32, device=dev))

    eager = bufs()
    run(*eager)
    torch.cuda.synchronize()
    graph_bufs = bufs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(*bufs())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(*graph_bufs)

    ref = [b.double().cpu().numpy() for b in eager[1:]]
    other = bufs()
    for rep in range(3):
        for b in graph_bufs:
            b.zero_()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("sum_delta", "state", "out", "last_state"), graph_bufs[1:],
                                   ref):
            check(f"graph {name} (replay {rep})", got.double().cpu().numpy(), want,
                  float(np.max(np.abs(want))), TOL["f32"])
        run(*other)                                  # eager work between replays
        torch.cuda.synchronize()
    check_device_errors(dev)
