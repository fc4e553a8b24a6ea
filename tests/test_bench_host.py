"""Host-side pieces of the benchmark that run without a GPU: the algorithmic
counts it reports and the CPU baseline on a pool of worker processes."""
import math

import bench
from synth import WORKLOADS, make_inputs


def test_algorithmic_counts_match_the_printed_budget():
    # the per-config budget table of the hot-path scope (F1 in GFLOP, Q2 in MB,
    # stage-2 flop per byte), as printed there to three figures
    printed = {"mid": (0.671, 68.2, 14.5), "long": (5.37, 142.6, 19.5),
               "s4d_lin": (2.15, 276.8, 17.0), "waveform": (10.74, 151.0, 21.9)}
    for name, (f1, q2, fpb) in printed.items():
        w = WORKLOADS[name]
        F1, Q2 = bench.algorithmic_counts(w)
        assert math.isclose(F1 / 1e9, f1, rel_tol=5e-3), name
        assert math.isclose(Q2 / 1e6, q2, rel_tol=5e-3), name
        assert math.isclose(bench.stage2_flops(w) / Q2, fpb, rel_tol=5e-3), name


def test_pool_baseline_splits_every_channel():
    x = make_inputs("tiny")
    r = bench.cpu_baseline_pool(x, max_workers=3)
    w = x["workload"]
    assert r["kind"] == "oracle" and r["unit"] == "samples/s"
    assert 1 <= r["cores"] <= min(3, w.H)
    assert r["value"] > 0 and r["seconds_per_forward"] > 0
