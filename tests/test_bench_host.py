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


def test_cpu_baseline_sample_and_parity_fields():
    # the GPU outputs replaced by the oracle's own: zero error, every field
    import numpy as np
    import oracle
    x = make_inputs("tiny")
    K, y = oracle.forward(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], x["D"], x["u"])
    cb, par = bench.cpu_baseline(x, K, y, min_seconds=0.0)
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["value"] > 0
    assert 1 <= par["channels_checked"] <= x["workload"].H
    assert par["K_max_rel_err"] == 0.0 and par["y_worst_channel_rel_err"] == 0.0


def test_roofline_picks_the_dominant_kernel():
    w = WORKLOADS["waveform"]
    r = bench.roofline(w, t_gen=190e-6, t_cauchy=130e-6, t_conv=136e-6)
    assert r["kernel"] == "cauchy_kernel" and r["bound"] == "alu" and r["unit"] == "TFLOP/s"
    assert math.isclose(r["frac"], bench.algorithmic_counts(w)[0] / 130e-6 / 1e12 / 157.3)
    assert r["conv"]["bound"] == "hbm" and "big_rows_pair_kernel" in r["conv"]["kernel"]
    m = WORKLOADS["mid"]
    r = bench.roofline(m, t_gen=16e-6, t_cauchy=20e-6, t_conv=26e-6)
    assert r["kernel"] == "conv_pair1024_kernel" and r["bound"] == "hbm"
    assert r["stage1_kernel"]["kernel"] == "kgen_wave_kernel"


def test_trace_and_counter_summaries(tmp_path):
    tr = tmp_path / "trace" / "host"
    tr.mkdir(parents=True)
    rows = [("void s4::cauchy_kernel<2, false>(s4::ParamPtrs, ...)", 0, 1000),
            ("void s4::cauchy_kernel<2, false>(s4::ParamPtrs, ...)", 5000, 7000),
            ("big_rows_pair_kernel(float2 const*, ...)", 8000, 8500)]
    with open(tr / "x_kernel_trace.csv", "w") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for n, a, b in rows:
            f.write(f'"{n}",{a},{b}\n')
    md = bench.summarize_trace(str(tmp_path / "trace"), "label", "cmd")
    assert "| cauchy_kernel | 2 | 1.50 |" in md and "| big_rows_pair_kernel | 1 | 0.50 |" in md
    for counter, val, copy in (("FETCH_SIZE", 100.0, 524288.0), ("WRITE_SIZE", 300.0, 1048576.0)):
        d = tmp_path / counter
        d.mkdir()
        with open(d / "r_counter_collection.csv", "w") as f:
            f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
            for i in range(6):
                f.write(f'{i},"s4::cauchy_kernel<2, false>(x)",{counter},{val}\n')
            f.write(f'9,"__amd_rocclr_copyBuffer",{counter},{copy}\n')
    res = bench.summarize_counters(str(tmp_path / "FETCH_SIZE"), str(tmp_path / "WRITE_SIZE"),
                                   "waveform", ["c1", "c2"])
    k = res["kernels"]["cauchy_kernel"]
    assert math.isclose(res["calibration"]["fetch_scale"], 2.0)
    assert math.isclose(k["bytes_per_launch"], 2.0 * 1024 * 100 + 1.0 * 1024 * 300)


def test_sq_summary(tmp_path):
    d = tmp_path / "sq"
    d.mkdir()
    with open(d / "r_counter_collection.csv", "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Grid_Size,Workgroup_Size,VGPR_Count,Scratch_Size,"
                "Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n")
        vals = {"SQ_INSTS_VALU": 2048.0, "GRBM_GUI_ACTIVE": 16.0, "SQ_WAVE_CYCLES": 100.0,
                "SQ_WAIT_ANY": 25.0, "SQ_WAIT_INST_LDS": 10.0, "SQ_INSTS_LDS": 7.0}
        for disp in (1, 2):   # the summary takes the kernel's last dispatch
            for k, v in vals.items():
                f.write(f'{disp},"void s4::cauchy_kernel<2, false, true>(x)",1024,256,36,0,{k},'
                        f'{v * disp},1000,{1000 + 2000 * disp}\n')
    md = bench.summarize_sq(str(d), "label", "cmd")
    # 2 x 2048 VALU instructions over 256 CUs x (2 x 16 / 8) cycles = 4.00 per CU-cycle
    assert "| cauchy_kernel | 1024 | 256 | 36 | 0 | 4.0 | 4.1e+03 | 4.00 | 14 | 0.25 | 0.10 |" in md
