"""Host-only checks of the benchmark's bookkeeping (no GPU): the roofline
arithmetic of a workload entry and the refusal of more than one GPU."""

import os
import subprocess
import sys

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_slot_and_transcendental_counts():
    # per state: mul, exp (2 slots), mul, fma, fma; per channel step 20
    assert bench.valu_slots_per_token_channel(16) == 116
    assert bench.valu_slots_per_token_channel(16, "zoh") == 276
    assert bench.transcendentals_per_token_channel(16) == 21


def test_forward_entry_fractions():
    w = synth.WORKLOADS["mamba2p8b"]
    ceil = {"fma_T_per_s": 35.0, "exp_T_per_s": 17.5}
    e = bench.fwd_entry(w, [0.8, 0.8, 0.8], ceil, traffic=1.4e9)
    tokch = 4 * 8192 * 5120
    assert e["tokens_channels_per_s"] == pytest.approx(tokch / 0.8e-3)
    nbytes = synth.algorithmic_bytes(w)
    assert e["algorithmic_bytes"] == nbytes == 1345953792
    assert e["hbm_frac_of_8TBps"] == pytest.approx(nbytes / 0.8e-3 / 8e12)
    assert e["alu"]["frac_of_nominal"] == pytest.approx(
        116 * tokch / 0.8e-3 / 1e12 / bench.VALU_PEAK_TSLOTS)
    assert e["alu"]["unit"] == "T VALU lane-slots/s"
    assert e["transcendentals"]["frac_of_measured_exp_rate"] == pytest.approx(
        21 * tokch / 0.8e-3 / 1e12 / 17.5)
    assert e["counter_traffic_over_algorithmic"] == pytest.approx(1.4e9 / nbytes)


def test_forward_entry_takes_the_region_average():
    w = synth.WORKLOADS["seq1m"]
    ceil = {"fma_T_per_s": 35.0, "exp_T_per_s": 17.5}
    e = bench.fwd_entry(w, [2.1, 2.0, 2.3], ceil, region_avg=1.95)
    tokch = w.batch * w.seqlen * w.dim
    assert e["avg_ms"] == 1.95 and e["tokens_channels_per_s"] == pytest.approx(tokch / 1.95e-3)
    assert e["per_call_avg_ms"] == pytest.approx(2.1333333) and e["median_ms"] == 2.1
    assert e["min_ms"] == 2.0 and "region" in e["timing"]


def test_nominal_valu_peak():
    # 256 CUs x 4 SIMD16 x 16 lanes x 2.4 GHz
    assert bench.VALU_PEAK_TSLOTS == pytest.approx(39.3216)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_compares_the_gpu_output_on_its_sample():
    """The baseline's oracle run doubles as a parity check of the GPU
    forward's output on the same prefix: an exact output reports zero error,
    a perturbed one its scaled error."""
    import oracle
    w = synth.WORKLOADS["tiny"]
    x = synth.make(w)
    dec = synth.make("decode", batch=32, dim=16, dstate=4)
    full, _ = oracle.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"],
                              x["dt_bias"])
    y, h = oracle.state_update(dec["state"], dec["u"], dec["delta"], dec["A"], dec["B"],
                               dec["C"], dec["D"], dec["z"], dec["dt_bias"])
    r = bench.cpu_baseline(x, w, dec, 0.01, gpu_out=full.astype("float32"),
                           gpu_dec=(y.astype("float32"), h.astype("float32")))
    p = r["gpu_forward_vs_oracle"]
    assert p["steps_compared"] >= 8 and p["max_abs_err_over_max_abs_out"] < 1e-6
    d = r["gpu_decode_vs_oracle"]
    assert d["out_max_abs_err_over_max_abs_out"] < 1e-6
    assert d["state_max_abs_err_over_max_abs_out"] < 1e-6
    bad = full.copy()
    bad[0, 0, 0] += 0.5 * abs(full).max()
    p2 = bench.cpu_baseline(x, w, dec, 0.01, gpu_out=bad)["gpu_forward_vs_oracle"]
    assert 0.4 < p2["max_abs_err_over_max_abs_out"] < 0.6


def test_backward_traffic_only_for_matching_counters():
    """The backward line's traffic comes from the committed counters of the
    2.8B training pair, only in that mode and with the kernel sources they
    were taken on; every other run reports none."""
    t = bench.bwd_traffic("mamba2p8b", True, "delta")
    assert t is not None and 4.7e9 < t < 6.0e9
    assert bench.bwd_traffic("mamba2p8b", False, "delta") is None
    assert bench.bwd_traffic("mamba2p8b", True, "zoh") is None
    assert bench.bwd_traffic("seq1m", True, "delta") is None
