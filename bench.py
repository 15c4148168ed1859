#!/usr/bin/env python3
"""Benchmark of the selective-scan hot path on one MI355X.

One step = one selective_scan_fwd over the Mamba-2.8B-shaped layer
(batch 4, L 8192, d_inner 5120, d_state 16, bfloat16 activations, float32
state and arithmetic) followed by one selective_state_update over the decode
workload (256 sequences x 5120 channels x 16 states).  Inputs are seeded
synthetic data (synth.make) already resident in HBM; decode states rotate
over six buffers (504 MB) so the 256 MB Infinity Cache cannot hold them
between steps.

Prints one JSON line.  `value` is tokens*channels processed per second over
the whole step (forward B*L*D plus decode B*D).  `roofline` describes the
forward kernel (the dominant one); `cpu_baseline` times the float64 oracle on
a bounded sample of the same workload on the host.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

# MI355X public figures: 256 CUs x 4 SIMD16 units at 2.4 GHz -> 39.3 T fp32
# vector lane-operations per second without packed math (the published
# 157.3 TFLOP/s counts an FMA as 2 flops and packed pairs as 2 lanes).
HBM_PEAK_GBS = 8000.0
# v_exp_f32 throughput measured on gfx950 with 4 waves per SIMD (half the
# FMA rate); the transcendental roofline of the forward
EXP_PEAK_TPS = 18.47
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12

METRIC = "selective-scan fwd tokens·channels/s and achieved HBM GB/s (% of peak), 1 GPU"


def valu_slots_per_token_channel(n, bbar="delta"):
    """Algorithmic fp32 VALU issue slots per token*channel of the forward:
    per state mul(Delta*A), exp, mul(Delta*u*B), fma(h), fma(y) = 6 slots with
    the transcendental at half rate (2 slots); per channel step softplus
    (exp, log, rcp + 5 ops = 11), gate (exp, rcp + 3 ops = 7), Delta*u and
    D*u (2): 20 slots.  The zero-order-hold input adds per state the
    coefficient (exp(Delta A) - 1)/A: a 5-term series and its scaling (6),
    the difference form (1), the choice between them (2) and one more
    product (1): 16 slots per state."""
    return (16 if bbar == "zoh" else 6) * n + 20


def bwd_valu_slots_per_token_channel(n):
    """Algorithmic fp32 VALU issue slots per token*channel of the backward
    with recomputation: per state the recomputed step and readout (mul, exp
    (2), mul, fma, fma = 6), the adjoint (lambda fma, dC and dB products,
    sum lambda B fma, Abar h_{t-1} and its product with lambda, sum with A,
    dA fma, the carried Abar lambda = 9) and the two channel sums of dB and
    dC (2): 17 slots; per channel step softplus and its derivative (14), the
    gate and its derivative (12), du and dDelta (4): 30 slots."""
    return 17 * n + 30


def bwd_algorithmic_bytes(w):
    """Reads u, dt, z, dout, B, C and the parameters; writes du, ddt, dz, dB,
    dC and the parameter gradients."""
    e = 2 if w.dtype == "bf16" else 4
    blD = w.batch * w.seqlen * w.dim
    blN = w.batch * w.seqlen * w.dstate
    params = 4 * (w.dim * w.dstate + 2 * w.dim)
    return 7 * e * blD + 4 * e * blN + 2 * params


def transcendentals_per_token_channel(n):
    """exp per state, plus exp/log/rcp of softplus and exp/rcp of the gate."""
    return n + 5


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="mamba2p8b",
                   choices=["mamba130m", "mamba2p8b", "seq1m"],
                   help="forward workload of the step (default: the 2.8B-shaped layer)")
    p.add_argument("--no-decode", action="store_true", help="time the forward alone")
    p.add_argument("--bbar", default="delta", choices=["delta", "zoh"],
                   help="input discretisation of forward and decode (default Delta*B)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate host time budget of the oracle baseline")
    p.add_argument("--bwd", action="store_true",
                   help="instead of the step: time the backward (selective_scan_bwd) on the "
                        "forward workload; one JSON line with its own roofline and CPU baseline")
    p.add_argument("--train", action="store_true",
                   help="with --bwd: the training pair (forward keeping checkpoints, then the "
                        "backward reading them)")
    p.add_argument("--conv", action="store_true",
                   help="instead of the step: time the causal conv1d + SiLU (width 4) on the "
                        "forward workload's activations; one JSON line with an HBM roofline")
    p.add_argument("--block", action="store_true",
                   help="instead of the step: time one Mamba block (projections, conv1d, scan) "
                        "of the workload's model with random weights; one JSON line")
    p.add_argument("--l-sweep", action="store_true",
                   help="instead of the step: time the forward alone over L = 2^10 .. 2^20 "
                        "at B=1, D=256, N=16, float32 (one JSON line per L)")
    p.add_argument("--copy-calibration-mb", type=int, default=0,
                   help="before timing, run one plain device copy of this many MiB "
                        "(a known-size reference for hardware byte counters)")
    return p.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_fwd_traffic_mamba2p8b.json")
KERNEL_SOURCES = [os.path.join(ROOT, "selective_state_space_38_amd", "csrc", f)
                  for f in ("scan_fwd.hip", "ssm_device.h", "ssm_internal.h", "api.hip")]


def kernel_source_digest():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per forward launch from the committed counter summary, or None
    when it was taken on another workload or the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(x, w, dec, budget_s, bbar="delta"):
    """Times the oracle (as it stands) on a bounded prefix of the workload:
    every batch row and channel, the first L' steps, L' sized to ~budget_s;
    plus one decode step on a 32-sequence slice of the decode workload."""
    import oracle

    def sample(L):
        sl = slice(0, L)
        return (x["u"][:, sl], x["delta"][:, sl], x["A"], x["B"][:, sl], x["C"][:, sl],
                x["D"], x["z"][:, sl], x["dt_bias"])

    t0 = time.perf_counter()
    oracle.scan_fwd(*sample(8), bbar=bbar)
    per_step = (time.perf_counter() - t0) / 8
    L = int(max(8, min(w.seqlen, budget_s / max(per_step, 1e-6))))
    t0 = time.perf_counter()
    oracle.scan_fwd(*sample(L), bbar=bbar)
    t_fwd = time.perf_counter() - t0
    nb = 32
    t0 = time.perf_counter()
    oracle.state_update(dec["state"][:nb], dec["u"][:nb], dec["delta"][:nb], dec["A"],
                        dec["B"][:nb], dec["C"][:nb], dec["D"], dec["z"][:nb],
                        dec["dt_bias"], bbar=bbar)
    t_dec = time.perf_counter() - t0
    tokch = w.batch * L * w.dim + nb * dec_dim(dec)
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - informational only
        blas_threads = None
    return {
        "value": tokch / (t_fwd + t_dec),
        "unit": "tokens·channels/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"float64 NumPy oracle, single-threaded ufuncs: forward on all {w.batch} "
                   f"batch rows and {w.dim} channels, first {L} of {w.seqlen} steps "
                   f"({t_fwd:.1f} s) + one decode step on {nb} sequences ({t_dec:.2f} s)"),
        "host_cpus_available": len(os.sched_getaffinity(0)),
        "blas_threads_idle": blas_threads,
    }


def dec_dim(dec):
    return dec["u"].shape[1]


def bwd_bench(args, torch, dev):
    """Times selective_scan_bwd on the workload's forward inputs with a
    seeded N(0,1) output gradient."""
    from selective_state_space_38_amd import (check_device_errors, ckpt_buffer,
                                              selective_scan_bwd, selective_scan_fwd)

    w = synth.WORKLOADS[args.workload]
    act = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    print(f"bench: generating {w.name} inputs", file=sys.stderr, flush=True)
    x = synth.make(w)
    dout_np = np.random.default_rng(w.seed + 100).standard_normal(x["u"].shape).astype(np.float32)
    if w.dtype == "bf16":
        dout_np = synth.round_bf16(dout_np)

    def up(a, dtype=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=dtype)

    u, dt, z, dout = up(x["u"], act), up(x["delta"], act), up(x["z"], act), up(dout_np, act)
    Bm, Cm = up(x["B"], act), up(x["C"], act)
    A, Dv, bias = up(x["A"]), up(x["D"]), up(x["dt_bias"])

    ck = ckpt_buffer(u, w.dstate) if args.train else None
    fout = torch.empty_like(u)

    def fwd_train():
        selective_scan_fwd(u, dt, A, Bm, Cm, D=Dv, z=z, delta_bias=bias, out=fout, ckpt=ck)

    if args.train:
        fwd_train()
        torch.cuda.synchronize()
        fwd_ms = _time_ms(torch, fwd_train, args.steps, args.warmup)

    def bwd():
        return selective_scan_bwd(u, dt, A, Bm, Cm, dout, D=Dv, z=z, delta_bias=bias, ckpt=ck)

    for _ in range(args.warmup):
        bwd()
    torch.cuda.synchronize()
    check_device_errors(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in ev:
        e[0].record()
        bwd()
        e[1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = [e[0].elapsed_time(e[1]) for e in ev]
    avg = float(np.mean(ms))
    tokch = w.batch * w.seqlen * w.dim
    slots = bwd_valu_slots_per_token_channel(w.dstate) * tokch
    achieved = slots / (avg / 1e3) / 1e12
    nbytes = bwd_algorithmic_bytes(w)
    line = {
        "metric": "selective-scan bwd tokens·channels/s, 1 GPU",
        "value": tokch / (avg / 1e3),
        "unit": "tokens·channels/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": (t1 - t0) * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded N(0,1) activations and output gradient)",
        "config": {"workload": (f"{w.name} backward (B={w.batch}, L={w.seqlen}, D={w.dim}, "
                                f"N={w.dstate}, {w.dtype} activations)"
                                + (", from the training-mode forward's checkpoints"
                                   if args.train else ", recomputing its own checkpoints"))},
        "roofline": {
            "bound": "alu", "achieved": achieved, "peak": VALU_PEAK_TOPS, "unit": "TFLOP/s",
            "frac": achieved / VALU_PEAK_TOPS, "traffic": None,
            "kernel": "scan_bwd_kernel (+ reductions)",
            "ops_per_unit": f"{bwd_valu_slots_per_token_channel(w.dstate)} fp32 VALU issue "
                            "slots per token*channel",
            "units_per_launch": tokch, "avg_launch_ms": avg,
            "median_launch_ms": float(np.median(ms)), "min_launch_ms": float(np.min(ms)),
        },
        "hbm": {"algorithmic_bytes": nbytes, "GBps": nbytes / (avg / 1e3) / 1e9,
                "frac_of_8TBps": nbytes / (avg / 1e3) / 1e9 / HBM_PEAK_GBS},
        "training_forward_ms": float(np.mean(fwd_ms)) if args.train else None,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        print("bench: timing the CPU oracle backward", file=sys.stderr, flush=True)

        def sample(Lp):
            sl = slice(0, Lp)
            return dict(u=x["u"][:, sl], delta=x["delta"][:, sl], A=x["A"], B=x["B"][:, sl],
                        C=x["C"][:, sl], D=x["D"], z=x["z"][:, sl], dt_bias=x["dt_bias"],
                        dout=dout_np[:, sl])

        t0 = time.perf_counter()
        oracle.scan_bwd(**sample(4))
        per_step = (time.perf_counter() - t0) / 4
        Lp = int(max(4, min(w.seqlen, args.cpu_seconds / max(per_step, 1e-6))))
        t0 = time.perf_counter()
        oracle.scan_bwd(**sample(Lp))
        tb = time.perf_counter() - t0
        line["cpu_baseline"] = {
            "value": w.batch * Lp * w.dim / tb, "unit": "tokens·channels/s", "cores": 1,
            "kind": "oracle",
            "sample": (f"float64 NumPy oracle backward, single-threaded ufuncs: all {w.batch} "
                       f"batch rows and {w.dim} channels, first {Lp} of {w.seqlen} steps "
                       f"({tb:.1f} s)"),
        }
    print(json.dumps(line), flush=True)


def conv_bench(args, torch, dev):
    """Times causal_conv1d_fwd (width 4, SiLU, bias, final state) over the
    workload's activation tensor; HBM-bound, so the roofline is bytes."""
    from selective_state_space_38_amd import causal_conv1d_fwd

    w = synth.WORKLOADS[args.workload]
    act = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    e = 2 if w.dtype == "bf16" else 4
    k = 4
    print(f"bench: generating {w.name} inputs", file=sys.stderr, flush=True)
    x_np = synth.make(w)["u"]
    r = np.random.default_rng(w.seed + 200)
    wt_np = (r.standard_normal((w.dim, k)) * 0.5).astype(np.float32)
    b_np = r.standard_normal(w.dim).astype(np.float32)
    x = torch.from_numpy(x_np).to(device=dev, dtype=act)
    wt = torch.from_numpy(wt_np).to(dev)
    bias = torch.from_numpy(b_np).to(dev)
    out = torch.empty_like(x)
    st = torch.empty((w.batch, w.dim, k - 1), dtype=torch.float32, device=dev)

    def conv():
        causal_conv1d_fwd(x, wt, bias, out=out, state_out=st, return_final_state=True)

    for _ in range(args.warmup):
        conv()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for ee in ev:
        ee[0].record()
        conv()
        ee[1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = [ee[0].elapsed_time(ee[1]) for ee in ev]
    avg = float(np.mean(ms))
    tokch = w.batch * w.seqlen * w.dim
    nbytes = 2 * e * tokch + 4 * (k * w.dim + w.dim) + 4 * w.batch * w.dim * (k - 1)
    gbps = nbytes / (avg / 1e3) / 1e9
    line = {
        "metric": "causal conv1d + SiLU tokens·channels/s and achieved HBM GB/s, 1 GPU",
        "value": tokch / (avg / 1e3), "unit": "tokens·channels/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": (t1 - t0) * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded N(0,1) activations and filters)",
        "config": {"workload": (f"{w.name} activations (B={w.batch}, L={w.seqlen}, "
                                f"D={w.dim}, {w.dtype}), width {k}")},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "conv1d_fwd_kernel", "bytes_per_launch": nbytes,
                     "avg_launch_ms": avg, "median_launch_ms": float(np.median(ms)),
                     "min_launch_ms": float(np.min(ms))},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        Lp = min(w.seqlen, 512)
        t0 = time.perf_counter()
        oracle.causal_conv1d(x_np[:, :Lp], wt_np, b_np)
        tb = time.perf_counter() - t0
        line["cpu_baseline"] = {
            "value": w.batch * Lp * w.dim / tb, "unit": "tokens·channels/s", "cores": 1,
            "kind": "oracle",
            "sample": (f"float64 NumPy oracle, single-threaded ufuncs: all {w.batch} batch rows "
                       f"and {w.dim} channels, first {Lp} of {w.seqlen} steps ({tb:.2f} s)"),
        }
    print(json.dumps(line), flush=True)


def _time_ms(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        fn()
        e[1].record()
    torch.cuda.synchronize()
    return [e[0].elapsed_time(e[1]) for e in ev]


def block_bench(args, torch, dev):
    """One Mamba block of the workload's model (B, L of the workload; d_model
    = d_inner / 2) with seeded random weights.  The conv1d and the scan are
    also timed alone on the same shapes, so the projections' share (hipBLASLt
    GEMMs on MFMA) is the block time minus theirs."""
    from selective_state_space_38_amd import (causal_conv1d_fwd, mamba_block_fwd,
                                              selective_scan_fwd)

    w = synth.WORKLOADS[args.workload]
    cfg = synth.BLOCKS[args.workload]
    act = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    print(f"bench: generating {w.name} block weights", file=sys.stderr, flush=True)
    x_np, wt_np = synth.make_block(**cfg, batch=w.batch, seqlen=w.seqlen, dtype=w.dtype)
    f32 = ("conv_w", "conv_b", "dt_bias", "A", "D")
    wt = {k: torch.from_numpy(v).to(device=dev, dtype=torch.float32 if k in f32 else act)
          for k, v in wt_np.items()}
    x = torch.from_numpy(x_np).to(device=dev, dtype=act)
    out = torch.empty_like(x)
    M = w.batch * w.seqlen
    dm, di, n, r = cfg["d_model"], cfg["d_inner"], cfg["d_state"], cfg["dt_rank"]
    ms_block = _time_ms(torch, lambda: mamba_block_fwd(x, wt, out=out), args.steps, args.warmup)
    # the block's own conv1d and scan, alone on the same shapes
    xi = torch.randn(w.batch, w.seqlen, di, device=dev).to(act)
    u = torch.empty_like(xi)
    ms_conv = _time_ms(torch, lambda: causal_conv1d_fwd(xi, wt["conv_w"], wt["conv_b"], out=u),
                       args.steps, args.warmup)
    dt = torch.randn(w.batch, w.seqlen, di, device=dev).to(act)
    Bm = torch.randn(w.batch, w.seqlen, n, device=dev).to(act)
    Cm = torch.randn(w.batch, w.seqlen, n, device=dev).to(act)
    y = torch.empty_like(xi)
    ms_scan = _time_ms(torch, lambda: selective_scan_fwd(u, dt, wt["A"], Bm, Cm, D=wt["D"], z=xi,
                                                         delta_bias=wt["dt_bias"], out=y),
                       args.steps, args.warmup)
    tb, tc, ts = (float(np.mean(v)) for v in (ms_block, ms_conv, ms_scan))
    gemm_flops = 2 * M * (dm * 2 * di + di * (r + 2 * n) + r * di + di * dm)
    t_gemm = max(tb - tc - ts, 1e-6)
    gemm_tflops = gemm_flops / (t_gemm / 1e3) / 1e12
    peak = 2500.0 if w.dtype == "bf16" else 157.3
    line = {
        "metric": "Mamba block forward tokens/s, 1 GPU",
        "value": M / (tb / 1e3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": tb,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype if w.dtype == "f32" else "bf16 storage, f32 accumulation",
        "data": "synthetic (seeded random weights and N(0,1) input)",
        "config": {"workload": (f"{w.name} block (B={w.batch}, L={w.seqlen}, d_model={dm}, "
                                f"d_inner={di}, d_state={n}, dt_rank={r}, conv width "
                                f"{cfg['conv_width']}, {w.dtype})")},
        "roofline": {"bound": "mfma", "achieved": gemm_tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": gemm_tflops / peak, "traffic": None,
                     "kernel": "projection GEMMs (block time minus conv1d and scan alone)",
                     "flops_per_launch": gemm_flops},
        "breakdown_ms": {"block": tb, "scan_alone": ts, "conv1d_alone": tc,
                         "projections_by_difference": t_gemm,
                         "block_median": float(np.median(ms_block)),
                         "block_min": float(np.min(ms_block))},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        Lp = 64
        t0 = time.perf_counter()
        oracle.mamba_block_fwd(x_np[:, :Lp], wt_np)
        tcpu = time.perf_counter() - t0
        line["cpu_baseline"] = {
            "value": w.batch * Lp / tcpu, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": (f"float64 NumPy oracle block on the first {Lp} tokens of every row "
                       f"({tcpu:.1f} s; the matrix products may use every host core)"),
        }
    print(json.dumps(line), flush=True)


def l_sweep(args, torch, dev):
    """Forward time against sequence length at the million-token shape's width:
    the work is linear in L, so tokens*channels/s should level off, not fall."""
    from selective_state_space_38_amd import check_device_errors, fwd_plan, selective_scan_fwd

    w = synth.WORKLOADS["seq1m"]
    print(f"bench: generating {w.name} inputs", file=sys.stderr, flush=True)
    x = synth.make(w)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=torch.float32)

    full = {k: up(x[k]) for k in ("u", "delta", "z", "B", "C")}
    A, Dv, bias = up(x["A"]), up(x["D"]), up(x["dt_bias"])
    for lg in range(10, 21):
        L = 1 << lg
        u, dt, z = (full[k][:, :L] for k in ("u", "delta", "z"))
        Bm, Cm = full["B"][:, :L], full["C"][:, :L]
        out = torch.empty_like(u)
        last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev)

        def fwd():
            selective_scan_fwd(u, dt, A, Bm, Cm, D=Dv, z=z, delta_bias=bias,
                               delta_softplus=True, return_last_state=True, out=out,
                               last_state=last)

        for _ in range(args.warmup):
            fwd()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
              for _ in range(args.steps)]
        for e in ev:
            e[0].record()
            fwd()
            e[1].record()
        torch.cuda.synchronize()
        check_device_errors(dev)
        ms = [e[0].elapsed_time(e[1]) for e in ev]
        med = float(np.median(ms))
        tokch = w.batch * L * w.dim
        slots = valu_slots_per_token_channel(w.dstate) * tokch
        print(json.dumps({
            "l_sweep": True, "batch": w.batch, "seqlen": L, "dim": w.dim, "dstate": w.dstate,
            "dtype": "f32", "median_ms": med, "min_ms": float(np.min(ms)),
            "tokens_channels_per_s": tokch / (med / 1e3),
            "alu_frac": slots / (med / 1e3) / 1e12 / VALU_PEAK_TOPS,
            "plan": fwd_plan(w.batch, L, w.dim, w.dstate, torch.float32),
        }), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this path runs on one GPU "
              "(no collectives, no sharding); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from selective_state_space_38_amd import (check_device_errors, fwd_plan,
                                              selective_scan_fwd, selective_state_update)

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.l_sweep:
        l_sweep(args, torch, dev)
        return
    if args.bwd:
        bwd_bench(args, torch, dev)
        return
    if args.conv:
        conv_bench(args, torch, dev)
        return
    if args.block:
        block_bench(args, torch, dev)
        return
    w = synth.WORKLOADS[args.workload]
    dw = synth.WORKLOADS["decode"]
    act = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dact = torch.bfloat16 if dw.dtype == "bf16" else torch.float32
    print(f"bench: generating {w.name} inputs", file=sys.stderr, flush=True)
    x = synth.make(w)
    dec = synth.make(dw)

    def up(a, dtype=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=dtype)

    # Input sets rotate when one set is small enough for the 256 MB Infinity
    # Cache to keep a useful share of it between steps (the 130M layer's 405
    # MB); the 2.8B layer (1.35 GB) and the million-token sequence (4.4 GB)
    # stream from HBM anyway.
    n_sets = 3 if synth.algorithmic_bytes(w) < 1 << 30 else 1
    sets = []
    for k in range(n_sets):
        xs = x if k == 0 else synth.make(w, seed=w.seed + 1000 * k)
        sets.append((up(xs["u"], act), up(xs["delta"], act), up(xs["z"], act),
                     up(xs["B"], act), up(xs["C"], act)))
    u = sets[0][0]
    A, Dv, bias = up(x["A"]), up(x["D"]), up(x["dt_bias"])
    out = torch.empty_like(u)
    last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev)
    n_rot = 6  # 6 x 84 MB of decode state: twice the 256 MB Infinity Cache
    states = [up(dec["state"]) for _ in range(n_rot)]
    dx, ddt, dz = up(dec["u"], dact), up(dec["delta"], dact), up(dec["z"], dact)
    dB, dC = up(dec["B"], dact), up(dec["C"], dact)
    dA, dD, dbias = up(dec["A"]), up(dec["D"]), up(dec["dt_bias"])
    dout = torch.empty_like(dx)
    torch.cuda.synchronize()
    if args.copy_calibration_mb > 0:
        nbytes = args.copy_calibration_mb << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"bench: copy calibration {nbytes} bytes read + {nbytes} bytes written",
              file=sys.stderr, flush=True)
        del src, dst

    fwd_calls = [0]

    def fwd():
        su, sdt, sz, sB, sC = sets[fwd_calls[0] % n_sets]
        fwd_calls[0] += 1
        selective_scan_fwd(su, sdt, A, sB, sC, D=Dv, z=sz, delta_bias=bias, delta_softplus=True,
                           return_last_state=True, out=out, last_state=last, bbar=args.bbar)

    def decode(i):
        selective_state_update(states[i % n_rot], dx, ddt, dA, dB, dC, D=dD, z=dz,
                               dt_bias=dbias, dt_softplus=True, out=dout, bbar=args.bbar)

    for i in range(args.warmup):
        fwd()
        if not args.no_decode:
            decode(i)
    torch.cuda.synchronize()
    check_device_errors(dev)
    print(f"bench: warmup done, timing {args.steps} steps", file=sys.stderr, flush=True)

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        fwd()
        ev[i][1].record()
        if not args.no_decode:
            decode(i)
        ev[i][2].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    check_device_errors(dev)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    fwd_ms = [e[0].elapsed_time(e[1]) for e in ev]
    dec_ms = [e[1].elapsed_time(e[2]) for e in ev]
    fwd_avg = float(np.mean(fwd_ms))
    dec_avg = float(np.mean(dec_ms))
    trans_rate = (transcendentals_per_token_channel(w.dstate) * w.batch * w.seqlen * w.dim
                  / (fwd_avg / 1e3) / 1e12)

    tokch_fwd = w.batch * w.seqlen * w.dim
    tokch_dec = 0 if args.no_decode else dw.batch * dw.dim
    value = (tokch_fwd + tokch_dec) / (ms_per_step / 1e3)
    fwd_bytes = synth.algorithmic_bytes(w)
    dec_bytes = synth.algorithmic_bytes(dw)
    slots = valu_slots_per_token_channel(w.dstate, args.bbar) * tokch_fwd
    achieved_t = slots / (fwd_avg / 1e3) / 1e12
    plan = fwd_plan(w.batch, w.seqlen, w.dim, w.dstate, act)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens·channels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) activations, S4D-real A, log-uniform dt bias)",
        "config": {
            "workload": (f"{w.name} forward (B={w.batch}, L={w.seqlen}, D={w.dim}, N={w.dstate}, "
                         f"{w.dtype} activations)"
                         + ("" if args.no_decode else
                            f" + decode update (B={dw.batch}, D={dw.dim}, N={dw.dstate}, "
                            f"{dw.dtype})")),
            "io_dtype": w.dtype,
            "bbar": args.bbar,
            "forward_plan": plan,
            "forward_input_sets": n_sets,
            "decode_state_sets": n_rot,
        },
        "roofline": {
            "bound": "alu",
            "achieved": achieved_t,
            "peak": VALU_PEAK_TOPS,
            "unit": "TFLOP/s",
            "frac": achieved_t / VALU_PEAK_TOPS,
            "traffic": measured_traffic(w.name) if args.bbar == "delta" else None,
            "kernel": "scan_fwd_kernel",
            "ops_per_unit": f"{valu_slots_per_token_channel(w.dstate, args.bbar)} fp32 VALU "
                            "issue slots per token*channel",
            "units_per_launch": tokch_fwd,
            "avg_launch_ms": fwd_avg,
            "median_launch_ms": float(np.median(fwd_ms)),
            "min_launch_ms": float(np.min(fwd_ms)),
            "transcendentals": {
                "per_token_channel": transcendentals_per_token_channel(w.dstate),
                "achieved_T_per_s": trans_rate,
                "measured_v_exp_peak_T_per_s": EXP_PEAK_TPS,
                "frac": trans_rate / EXP_PEAK_TPS,
            },
        },
        "hbm": {
            "forward_GBps": fwd_bytes / (fwd_avg / 1e3) / 1e9,
            "forward_frac_of_8TBps": fwd_bytes / (fwd_avg / 1e3) / 1e9 / HBM_PEAK_GBS,
            "forward_algorithmic_bytes": fwd_bytes,
            "decode_GBps": (None if args.no_decode else
                            dec_bytes / (dec_avg / 1e3) / 1e9),
            "decode_frac_of_8TBps": (None if args.no_decode else
                                     dec_bytes / (dec_avg / 1e3) / 1e9 / HBM_PEAK_GBS),
            "decode_algorithmic_bytes": dec_bytes,
            "decode_avg_launch_ms": None if args.no_decode else dec_avg,
            "decode_median_launch_ms": None if args.no_decode else float(np.median(dec_ms)),
            "decode_min_launch_ms": None if args.no_decode else float(np.min(dec_ms)),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(x, w, dec, args.cpu_seconds, args.bbar)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
