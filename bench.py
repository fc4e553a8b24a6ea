#!/usr/bin/env python3
"""Throughput of the S4 DPLR convolution-mode forward pass on one MI355X.

One step = one call of the library's fused forward entry point over one batch
of synthetic input: pole packing, the Cauchy/Woodbury kernel generation, the
kernel spectrum (inverse FFT to K, which is written out, and the zero-padded
2L spectrum) and the causal FFT convolution with the D skip, y = K * u + D u.

Prints ONE JSON line on stdout; progress goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mid]

Inputs are resident in HBM before the timed region.  The timed steps rotate
over several input/output buffer sets whose total exceeds 512 MB so that the
256 MB last-level cache does not hold a step's data from the previous step.
After the K timed steps the two stages are timed separately with HIP events
on the launch stream: kernel generation alone, and the convolution kernel
alone (``conv_apply``: one launch of the convolution kernel per step) -- the
latter gives the roofline figure.  The CPU baseline runs the fp64 oracle on
the host on the same workload, on one thread and split over channels across
a pool of worker processes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "S4 conv fwd samples/s (B·H·L/s) + Cauchy kernel-gen GFLOP/s vs fp32 peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "conv_traffic.json")
KERNEL_SOURCES = ["kernels.hip", "device_fft.h", "fft_sched.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "structured_state_space_dplr_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_counts(w):
    """Algorithmic work of one forward pass (not the work the method avoids).

    F1: Cauchy stage flops, H*L*N*(8 + 8*S) with S = 4 sums (DPLR) or 1
        (diagonal): 8 flops per complex reciprocal, 8 per complex
        multiply-accumulate.
    Q2: convolution bytes, 4 B*H*L (read u) + 4 B*H*L (write y) + 4 H*L
        (the kernel) + 4 H (D).
    """
    S = 1 if w.diagonal else 4
    F1 = w.H * w.L * w.N * (8 + 8 * S)
    Q2 = 8 * w.batch * w.H * w.L + 4 * w.H * w.L + 4 * w.H
    return F1, Q2


def stage2_flops(w):
    """Convolution flops, for the VALU cross-check only: B*H*(5*2L*log2(2L) +
    6(L+1)) for the transforms of u and y and the bin products, plus
    H*2.5*2L*log2(2L) for the kernel spectrum."""
    import math
    n2 = 2 * w.L
    lg = math.log2(n2)
    return w.batch * w.H * (5 * n2 * lg + 6 * (w.L + 1)) + w.H * 2.5 * n2 * lg


def recurrent_counts(w):
    """Algorithmic work of the recurrent view (O(N) bilinear DPLR step).

    Flops per pole per step: the update w = Abar0 x - e qx + Bbar0 u (two
    complex products, one real-by-complex product, two complex adds: 18),
    x' = w - g qw (8), the output Re(C x') accumulated (4), and the two sums
    conj(Q) x' and qa x' for the next step (16): 46.  Diagonal: Abar0 x +
    Bbar0 u (10) and the output (4): 14.
    Bytes of one decode step (T = 1): the state read and written (16 B per
    pole), u read and y written (8 B per sequence).
    """
    per_pole = 14 if w.diagonal else 46
    rows = w.batch * w.H
    return per_pole * w.N * rows, 16 * w.N * rows + 8 * rows


def backward_counts(w):
    """Algorithmic work of the backward pass.

    conv_bwd bytes: u, dy read and du written once each (4 B per sample),
    K read and dK written (4 B per (h, k)), D and dD.
    kernel_gen_bwd flops per (h, l, n): the forward Cauchy sums recomputed
    for the Woodbury partials (40 DPLR / 16 diagonal, as in the forward) and
    the transposed per-pole sums: the reciprocal (8), the sums R_ab (8 per
    complex multiply-add: 32 DPLR / 8 diagonal), sum_ab conj(w_ab) beta_ab
    (32 / 8), conj(r)^2 (6), t = conj(r)^2 m (6), T += t (2), E += conj(g) t (4).
    """
    bhl, hl = w.batch * w.H * w.L, w.H * w.L
    q_conv = 12 * bhl + 8 * hl + 8 * w.H
    per_term = (16 + 8 + 8 + 8 + 18) if w.diagonal else (40 + 8 + 32 + 32 + 18)
    return q_conv, w.H * w.L * w.N * per_term


def conv_kernel_name(L: int) -> str:
    """The kernel(s) that apply the convolution at sequence length L."""
    if L == 1024:
        return "conv_pair1024_kernel (one row per wave, paired lanes, one launch per step)"
    if 32 <= L <= 512:
        return "conv_wave_kernel (one row per wave, one launch per step)"
    if 2048 <= L <= 16384:
        return "conv_rows_kernel (one row per workgroup, one launch per step)"
    if L >= 32768:
        return ("big_cols_fwd_kernel + big_rows_pair_kernel + big_cols_inv_kernel "
                "(four-step transform, three launches per step)")
    return "conv_kernel (halves formulation, one launch per step)"


def read_traffic(workload_name: str):
    """HBM bytes per convolution launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload_name or t.get("kernel_source_sha") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(x, K_gpu, y_gpu, min_seconds: float):
    """The fp64 oracle (the pages' Cauchy/Woodbury method and an fp64 FFT
    convolution) on the whole workload, one BLAS thread, repeated until
    `min_seconds` of CPU work; also the GPU result's error against it."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    w = x["workload"]
    times = []
    with threadpool_limits(1):
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            K, y = oracle.forward(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], x["D"],
                                  x["u"], method="cauchy", diagonal=w.diagonal)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start >= min_seconds and len(times) >= 3:
                break
    t = statistics.median(times)
    samples = w.batch * w.H * w.L
    eK = float(np.abs(K_gpu - K).max() / np.abs(K).max())
    ey = float(np.abs(y_gpu - y).max() / np.abs(y).max())
    return {
        "value": samples / t, "unit": "samples/s", "cores": 1, "kind": "oracle",
        "sample": (f"whole {w.name} workload (H={w.H}, N={w.N}, L={w.L}, batch={w.batch}), "
                   f"fp64 NumPy oracle: Cauchy/Woodbury kernel + rfft convolution; "
                   f"median of {len(times)} runs, 1 thread"),
        "seconds_per_forward": t,
    }, {"K_max_rel_err": eK, "y_max_rel_err": ey, "tolerance": 1e-4,
        "reference": "fp64 oracle, same seeded inputs"}


_POOL_X = None


def _pool_part(hs):
    """One worker's share of the pool baseline: the oracle forward on channels
    hs[0]:hs[1] of the inputs inherited from the parent, one BLAS thread."""
    from threadpoolctl import threadpool_limits

    import oracle

    x = _POOL_X
    sl = slice(hs[0], hs[1])
    cut = lambda a: None if a is None else a[sl]
    with threadpool_limits(1):
        oracle.forward(x["lam"][sl], cut(x["P"]), cut(x["Q"]), x["B"][sl], x["C"][sl],
                       x["dt"][sl], x["D"][sl], x["u"][:, sl], method="cauchy",
                       diagonal=x["workload"].diagonal)
    return hs


def cpu_baseline_pool(x, max_workers: int = 16):
    """The same oracle forward split over channels across a pool of worker
    processes (fork, one BLAS thread each): the median of 3 timed runs after
    one warm-up.  Workers never touch the GPU."""
    import multiprocessing as mp

    global _POOL_X
    w = x["workload"]
    P = max(1, min(max_workers, len(os.sched_getaffinity(0)), w.H))
    bounds = [(w.H * i // P, w.H * (i + 1) // P) for i in range(P)]
    _POOL_X = x
    times = []
    with mp.get_context("fork").Pool(P) as pool:
        pool.map(_pool_part, bounds)
        for _ in range(3):
            t0 = time.perf_counter()
            pool.map(_pool_part, bounds)
            times.append(time.perf_counter() - t0)
    _POOL_X = None
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    t = statistics.median(times)
    return {"value": w.batch * w.H * w.L / t, "unit": "samples/s", "cores": P, "kind": "oracle",
            "sample": (f"whole {w.name} workload split over channels across {P} worker "
                       f"processes (fp64 NumPy oracle, one thread each); median of 3 runs"),
            "cpu_model": model, "seconds_per_forward": t}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mid",
                    help="tiny | mid | long | s4d_lin | waveform (default: mid)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration runs)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported: the channels shard across GPUs with no exchange, so the figure of "
              "interest is the one-GPU throughput at the full workload shape.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import structured_state_space_dplr_amd as s4
    from synth import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    w = WORKLOADS[args.workload]
    log(f"[bench] workload {w.describe()}; generating inputs")
    x = make_inputs(w.name)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def g(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    params = {k: g(x[k]) for k in ("lam", "P", "Q", "B", "C", "dt", "D")}
    u0 = g(x["u"])
    row_bytes = 4 * w.batch * w.H * w.L
    nsets = min(1024, max(2, -(-(512 << 20) // (2 * row_bytes)) + 1))
    us = [u0] + [u0.clone() for _ in range(nsets - 1)]
    ys = [torch.empty_like(u0) for _ in range(nsets)]
    K = torch.empty((w.H, w.L), dtype=torch.float32, device=dev)
    plan = s4.Plan(w.H, w.N, w.L, w.batch, diagonal=w.diagonal, device=dev)
    ws = plan.workspace()
    stream = torch.cuda.current_stream()
    P = None if w.diagonal else params["P"]

    def step(i):
        s4.forward(plan, params["lam"], P, params["Q"], params["B"], params["C"], params["dt"],
                   params["D"], us[i % nsets], K, ys[i % nsets], ws, stream)

    log(f"[bench] {nsets} buffer sets of {2 * row_bytes / 2**20:.1f} MiB; warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # ---- timed region: exactly K forward steps ---------------------------------
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms_events = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = 1e3 * wall / args.steps
    samples = w.batch * w.H * w.L
    value = samples / (wall / args.steps)
    log(f"[bench] forward: {ms_per_step * 1e3:.1f} us/step (events {fwd_ms_events * 1e3:.1f} us)")
    # the same steps once more, each between its own events: median and minimum
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    per_step_us = [a.elapsed_time(b) * 1e3 for a, b in evs]
    fwd_med_us, fwd_min_us = statistics.median(per_step_us), min(per_step_us)
    log(f"[bench] forward per step: median {fwd_med_us:.1f} us, minimum {fwd_min_us:.1f} us")

    # keep the first set's outputs for the parity check against the oracle
    step(0)
    torch.cuda.synchronize()
    K_gpu = K.cpu().numpy().astype(np.float64)
    y_gpu = ys[0].cpu().numpy().astype(np.float64)

    # ---- stage 1 alone: kernel generation (pack, Cauchy, kernel spectrum) ------
    def timed(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(n):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e-3       # seconds per call

    t_gen = timed(lambda i: s4.kernel_gen(plan, params["lam"], P, params["Q"], params["B"],
                                          params["C"], params["dt"], K, ws, stream), args.steps)
    # ---- stage 2 alone: one convolution-kernel launch per call ------------------
    step(0)    # leaves the spectrum of this layer (with D) in the workspace
    t_conv = timed(lambda i: s4.conv_apply(plan, us[i % nsets], ys[i % nsets], ws, stream),
                   args.steps)
    F1, Q2 = algorithmic_counts(w)
    log(f"[bench] kernel_gen {t_gen * 1e6:.1f} us ({F1 / t_gen / 1e9:.0f} GFLOP/s), "
        f"conv {t_conv * 1e6:.1f} us ({Q2 / t_conv / 1e9:.0f} GB/s)")

    # ---- the recurrent view: a full scan (T = L) and one decode step (T = 1) ---
    flops_step, decode_bytes = recurrent_counts(w)
    s4.recurrent_prepare(plan, params["lam"], P, params["Q"], params["B"], params["C"],
                         params["dt"], ws, stream)
    state = torch.zeros((w.batch, w.H, w.N, 2), dtype=torch.float32, device=dev)
    scan = lambda i: s4.recurrent_scan(plan, params["D"], us[i % nsets], state, ys[i % nsets],
                                       ws, stream)
    t_one = timed(scan, 1)
    n_scan = max(3, min(args.steps, int(0.5 / max(t_one, 1e-6))))
    t_scan = timed(scan, n_scan)
    u1 = us[0][..., :1].contiguous()
    y1 = torch.empty_like(u1)
    t_dec = timed(lambda i: s4.recurrent_scan(plan, params["D"], u1, state, y1, ws, stream), 200)
    rec_tflops = flops_step * w.L / t_scan / 1e12
    log(f"[bench] recurrent scan {t_scan * 1e6:.1f} us ({samples / t_scan:.3g} samples/s, "
        f"{rec_tflops:.1f} TFLOP/s); decode step {t_dec * 1e6:.2f} us")

    # ---- zero-order hold (diagonal): the Vandermonde kernel on the same poles ---
    zplan = s4.Plan(w.H, w.N, w.L, w.batch, diagonal=True, zoh=True, device=dev)
    zws = zplan.workspace()
    t_vd = timed(lambda i: s4.kernel_gen(zplan, params["lam"], None, None, params["B"],
                                         params["C"], params["dt"], K, zws, stream), args.steps)
    f_vd = 7 * w.H * w.L * w.N      # per (h, k, n): one complex product and one add
    log(f"[bench] zoh kernel_gen {t_vd * 1e6:.1f} us ({f_vd / t_vd / 1e9:.0f} GFLOP/s)")
    zoh = {"kernel_gen_us": t_vd * 1e6, "gflops": f_vd / t_vd / 1e9,
           "frac_fp32_peak": f_vd / t_vd / 1e12 / FP32_PEAK_TFLOPS, "algorithmic_flops": f_vd,
           "note": "Vandermonde kernel plus the spectrum of K padded to 2L"}
    zplan.close()

    # ---- the block around the layer: layer norm, the layer, GLU projection ------
    from synth import make_block_params
    bp = {k: g(v) for k, v in make_block_params(w.H, seed=1).items()}
    bplan = s4.Plan(w.H, w.N, w.L, w.batch, diagonal=w.diagonal, device=dev, block=True)
    bws = bplan.workspace()
    t_blk = timed(lambda i: s4.block_forward(
        bplan, us[i % nsets], bp["gamma"], bp["beta"], params["lam"], P, params["Q"],
        params["B"], params["C"], params["dt"], params["D"], bp["W"], bp["bias"],
        ys[i % nsets], bws, stream), args.steps)
    f_proj = 2 * (2 * w.H) * w.H * w.batch * w.L        # the projection GEMM
    log(f"[bench] block forward {t_blk * 1e6:.1f} us ({samples / t_blk:.3g} samples/s; "
        f"projection {f_proj / 1e9:.2f} GFLOP)")
    block = {"us": t_blk * 1e6, "samples_per_s": samples / t_blk,
             "projection_flops": f_proj,
             "note": "layer norm + layer + GLU projection with residual (bf16 MFMA on hi/lo split operands, fp32 accumulation)"}
    bplan.close()

    # ---- the backward pass: conv_bwd and kernel_gen_bwd -----------------------
    bwd = None
    if True:
        q_bwd, f_bwd = backward_counts(w)
        dy = ys[1 % nsets]
        du = ys[2 % nsets]
        dK = torch.empty((w.H, w.L), dtype=torch.float32, device=dev)
        dD = torch.empty((w.H,), dtype=torch.float32, device=dev)
        grads = {k: torch.empty((w.H, w.N, 2), dtype=torch.float32, device=dev)
                 for k in ("lam", "P", "B", "C")}
        ddt = torch.empty((w.H,), dtype=torch.float32, device=dev)
        t_cb = timed(lambda i: s4.conv_bwd(plan, us[i % nsets], K, params["D"], dy, du, dK, dD,
                                           ws, stream), args.steps)
        t_kb = timed(lambda i: s4.kernel_gen_bwd(
            plan, params["lam"], P, params["Q"], params["B"], params["C"], params["dt"], dK,
            grads["lam"], None if w.diagonal else grads["P"], None, grads["B"], grads["C"], ddt,
            ws, stream), args.steps)
        log(f"[bench] conv_bwd {t_cb * 1e6:.1f} us ({q_bwd / t_cb / 1e9:.0f} GB/s), "
            f"kernel_gen_bwd {t_kb * 1e6:.1f} us ({f_bwd / t_kb / 1e9:.0f} GFLOP/s)")
        bwd = {
            "conv_bwd_us": t_cb * 1e6,
            "conv_bwd_gbs": q_bwd / t_cb / 1e9,
            "conv_bwd_frac_hbm": q_bwd / t_cb / 1e9 / HBM_PEAK_GBS,
            "conv_bwd_algorithmic_bytes": q_bwd,
            "kernel_gen_bwd_us": t_kb * 1e6,
            "kernel_gen_bwd_gflops": f_bwd / t_kb / 1e9,
            "kernel_gen_bwd_frac_fp32_peak": f_bwd / t_kb / 1e12 / FP32_PEAK_TFLOPS,
            "kernel_gen_bwd_algorithmic_flops": f_bwd,
            "samples_per_s": samples / (t_cb + t_kb),
        }

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 5 copies of 1 GiB done")

    traffic = read_traffic(w.name)
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "H": w.H, "N": w.N, "L": w.L, "batch": w.batch,
                   "init": w.init, "u": w.u_kind, "seed": 0},
        "roofline": {
            "kernel": conv_kernel_name(w.L),
            "bound": "hbm",
            "achieved": Q2 / t_conv / 1e9,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": Q2 / t_conv / 1e9 / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": Q2,
            "launch_us": t_conv * 1e6,
            "valu_frac_fp32_peak": stage2_flops(w) / t_conv / 1e12 / FP32_PEAK_TFLOPS,
        },
        "kernel_gen": {
            "us": t_gen * 1e6,
            "gflops": F1 / t_gen / 1e9,
            "frac_fp32_peak": F1 / t_gen / 1e12 / FP32_PEAK_TFLOPS,
            "algorithmic_flops": F1,
            "note": "pack + Cauchy/Woodbury + kernel spectrum; flops counted for the Cauchy sums",
        },
        "recurrent": {
            "kernel": "recurrent_scan_kernel (O(N) bilinear DPLR step, carried state)",
            "scan_us": t_scan * 1e6,
            "scan_samples_per_s": samples / t_scan,
            "bound": "alu",
            "achieved": rec_tflops,
            "peak": FP32_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": rec_tflops / FP32_PEAK_TFLOPS,
            "algorithmic_flops_per_step": flops_step,
            "decode_step_us": t_dec * 1e6,
            "decode_bytes_per_step": decode_bytes,
            "decode_tokens_per_s": w.batch / t_dec,
        },
        "backward": bwd,
        "zoh": zoh,
        "block": block,
        "forward_us_events": fwd_ms_events * 1e3,
        "forward_us_median": fwd_med_us,
        "forward_us_min": fwd_min_us,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"[bench] CPU baseline: fp64 oracle, >= {args.cpu_seconds:.0f} s")
        cb, parity = cpu_baseline(x, K_gpu, y_gpu, args.cpu_seconds)
        result["cpu_baseline"] = cb
        result["parity"] = parity
        log(f"[bench] oracle {cb['value']:.3g} samples/s; parity K {parity['K_max_rel_err']:.2e} "
            f"y {parity['y_max_rel_err']:.2e}")
        cp = cpu_baseline_pool(x)
        result["cpu_baseline_pool"] = cp
        log(f"[bench] oracle on {cp['cores']} worker processes: {cp['value']:.3g} samples/s "
            f"({cp['cpu_model']})")
    plan.close()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
