#!/usr/bin/env python3
"""Throughput of the S4 DPLR convolution-mode forward pass on one MI355X.

One step = one call of the library's fused forward entry point over one batch
of synthetic input: pole packing, the Cauchy/Woodbury kernel generation, the
kernel spectrum (inverse FFT to K, which is written out, and the zero-padded
2L spectrum) and the causal FFT convolution with the D skip, y = K * u + D u.

Prints ONE JSON line on stdout; progress goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload waveform]
                  [--configs all|none|name,name,...]

The headline workload is the largest single-GPU one (waveform: H = 64, N = 64,
L = 65536, batch = 4, the most work per step).  ``value`` is its whole-step
throughput, B*H*L samples per second.  The same line carries a ``configs``
map with the forward, stage-1 and convolution figures of every workload.

Inputs are resident in HBM before the timed region.  The timed steps rotate
over several input/output buffer sets totalling more than 512 MB, so that the
256 MB last-level cache does not hold a step's data from the previous step
(the tiny workload's sets are capped at 1024 and stay cache-resident; that
workload is launch-bound).  After the K timed steps each stage is timed alone
with HIP events on the launch stream: kernel generation (stage 1), the
generating function alone (the Cauchy kernel), and the convolution
(``conv_apply``).  By default K = 50 timed steps after W = 5 warmup steps,
and the per-step median and minimum come from K more steps, each between its
own pair of events.  The CPU baseline runs the fp64 oracle on the host on a
bounded sample of the headline workload (a subset of its channels, every
batch row), on one thread and over a pool of worker processes.

Three more modes turn rocprofv3 output into the summaries under ``profiles/``:
  python bench.py --summarize-trace DIR --label NAME --command CMD
  python bench.py --summarize-counters FETCH_DIR WRITE_DIR --workload NAME --command CMD
  python bench.py --summarize-sq DIR --workload NAME --command CMD
and ``--counters`` runs the short, fixed launch sequence those counter runs
profile; each summary records the rocprofv3 command that produced it.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "S4 conv fwd samples/s (B·H·L/s) + Cauchy kernel-gen GFLOP/s vs fp32 peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector, published: 256 CU x 4 SIMD x 2.4 GHz x 64 flop/clk
HEADLINE = "waveform"
ALL_CONFIGS = ["tiny", "mid", "long", "s4d_lin", "waveform"]
PROFILES = os.path.join(ROOT, "profiles")
# sources whose change makes a recorded counter figure stale
KERNEL_SOURCES = ["kernels.hip", "big.hip", "cauchy.h", "device_fft.h", "fft_sched.h"]


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
    (32 / 8), conj(r)^2 (6), t = conj(r)^2 m (6), T += t (2).  (dt comes from
    the per-pole gradients, not from a frequency sum.)
    """
    bhl, hl = w.batch * w.H * w.L, w.H * w.L
    q_conv = 12 * bhl + 8 * hl + 8 * w.H
    per_term = (16 + 8 + 8 + 8 + 14) if w.diagonal else (40 + 8 + 32 + 32 + 14)
    return q_conv, w.H * w.L * w.N * per_term


def fused_stage1(L: int) -> bool:
    return 32 <= L <= 1024


def stage1_kernel_name(L: int) -> str:
    if fused_stage1(L):
        return "kgen_wave_kernel"
    return "cauchy_kernel"


def conv_kernel_names(L: int) -> list[str]:
    """The kernel(s) that apply the convolution at sequence length L."""
    if L == 1024:
        return ["conv_pair1024_kernel"]
    if 32 <= L <= 512:
        return ["conv_wave_kernel"]
    if 2048 <= L <= 16384:
        return ["conv_rows_kernel"]
    if L >= 32768:
        return ["big_cols_fwd_kernel", "big_rows_pair_kernel", "big_cols_inv_kernel"]
    return ["conv_kernel"]


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"traffic_{workload}.json")


def read_traffic(workload: str):
    """HBM bytes per launch by kernel from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources; else {}."""
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    if t.get("kernel_source_sha") != kernel_source_hash():
        return {}
    return {k: v["bytes_per_launch"] for k, v in t.get("kernels", {}).items()}


# ---------------------------------------------------------------------------
# CPU baseline (the oracle): the only leg that touches oracle/
# ---------------------------------------------------------------------------

def _oracle_forward(x, hs):
    import oracle
    sl = slice(hs[0], hs[1])
    cut = lambda a: None if a is None else a[sl]
    return oracle.forward(x["lam"][sl], cut(x["P"]), cut(x["Q"]), x["B"][sl], x["C"][sl],
                          x["dt"][sl], x["D"][sl], x["u"][:, sl], method="cauchy",
                          diagonal=x["workload"].diagonal)


def cpu_baseline(x, K_gpu, y_gpu, min_seconds: float):
    """The fp64 oracle (the pages' Cauchy/Woodbury method and an fp64 FFT
    convolution) on a bounded sample of the workload: the first `hs` channels
    with every batch row, `hs` chosen so that one run takes about 2 s; one
    BLAS thread, repeated until `min_seconds` of CPU work.  Also the GPU
    result's error against it on those channels (whole sample and worst
    channel)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    w = x["workload"]
    with threadpool_limits(1):
        t0 = time.perf_counter()
        _oracle_forward(x, (0, 1))
        t1 = time.perf_counter() - t0
        hs = max(1, min(w.H, int(2.0 / max(t1, 1e-3))))
        times = []
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            K, y = _oracle_forward(x, (0, hs))
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start >= min_seconds and len(times) >= 3:
                break
    t = statistics.median(times)
    samples = w.batch * hs * w.L
    Kg, yg = K_gpu[:hs], y_gpu[:, :hs]
    eK = float(np.abs(Kg - K).max() / np.abs(K).max())
    ey = float(np.abs(yg - y).max() / np.abs(y).max())
    cK = np.abs(Kg - K).max(axis=1) / np.abs(K).max(axis=1)
    cy = np.abs(yg - y).max(axis=(0, 2)) / np.abs(y).max(axis=(0, 2))
    return {
        "value": samples / t, "unit": "samples/s", "cores": 1, "kind": "oracle",
        "sample": (f"{w.name} workload, channels 0..{hs - 1} of {w.H} with all {w.batch} batch "
                   f"rows (B*{hs}*L = {samples} samples per run), fp64 NumPy oracle: "
                   f"Cauchy/Woodbury kernel + rfft convolution; median of {len(times)} runs, "
                   f"1 thread"),
        "seconds_per_run": t,
    }, {"K_max_rel_err": eK, "y_max_rel_err": ey,
        "K_worst_channel_rel_err": float(cK.max()), "y_worst_channel_rel_err": float(cy.max()),
        "channels_checked": hs, "tolerance": 1e-4,
        "reference": "fp64 oracle, same seeded inputs"}


_POOL_X = None


def _pool_part(hs):
    """One worker's share of the pool baseline: the oracle forward on channels
    hs[0]:hs[1] of the inputs inherited from the parent, one BLAS thread."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        _oracle_forward(_POOL_X, hs)
    return hs


def cpu_baseline_pool(x, max_workers: int = 16):
    """The same oracle forward on the whole workload, split over channels
    across a pool of worker processes (fork, one BLAS thread each): the median
    of 3 timed runs after one warm-up.  The pool has min(16, affinity, H)
    workers: 16 is the host's CPU share per GPU.  Workers never touch the GPU."""
    import multiprocessing as mp

    global _POOL_X
    w = x["workload"]
    affinity = len(os.sched_getaffinity(0))
    P = max(1, min(max_workers, affinity, w.H))
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
                       f"processes (fp64 NumPy oracle, one thread each; {affinity} cores in "
                       f"the affinity mask, capped at 16); median of 3 runs"),
            "cpu_model": model, "seconds_per_forward": t}


# ---------------------------------------------------------------------------
# GPU measurement of one workload
# ---------------------------------------------------------------------------

class Workbench:
    """Inputs, rotating buffer sets, plan and workspace of one workload."""

    def __init__(self, s4, torch, w, dev):
        import numpy as np

        from synth import make_inputs
        self.s4, self.torch, self.w, self.dev = s4, torch, w, dev
        self.x = make_inputs(w.name)
        g = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        self.params = {k: g(self.x[k]) for k in ("lam", "P", "Q", "B", "C", "dt", "D")}
        self.P = None if w.diagonal else self.params["P"]
        u0 = g(self.x["u"])
        row_bytes = 4 * w.batch * w.H * w.L
        self.nsets = min(1024, max(2, -(-(512 << 20) // (2 * row_bytes)) + 1))
        self.set_mib = 2 * row_bytes / 2 ** 20
        self.us = [u0] + [u0.clone() for _ in range(self.nsets - 1)]
        self.ys = [torch.empty_like(u0) for _ in range(self.nsets)]
        self.K = torch.empty((w.H, w.L), dtype=torch.float32, device=dev)
        self.khat = torch.empty((w.H, w.L, 2), dtype=torch.float32, device=dev)
        self.plan = s4.Plan(w.H, w.N, w.L, w.batch, diagonal=w.diagonal, device=dev)
        self.ws = self.plan.workspace()
        self.stream = torch.cuda.current_stream()

    def step(self, i):
        p = self.params
        self.s4.forward(self.plan, p["lam"], self.P, p["Q"], p["B"], p["C"], p["dt"], p["D"],
                        self.us[i % self.nsets], self.K, self.ys[i % self.nsets], self.ws,
                        self.stream)

    def kernel_gen(self, i):
        p = self.params
        self.s4.kernel_gen(self.plan, p["lam"], self.P, p["Q"], p["B"], p["C"], p["dt"], self.K,
                           self.ws, self.stream)

    def cauchy(self, i):
        p = self.params
        self.s4.generating_function(self.plan, p["lam"], self.P, p["Q"], p["B"], p["C"], p["dt"],
                                    self.khat, self.ws, self.stream)

    def conv(self, i):
        self.s4.conv_apply(self.plan, self.us[i % self.nsets], self.ys[i % self.nsets], self.ws,
                           self.stream)

    def timed(self, fn, n, warm=3):
        """Seconds per call: n calls between two HIP events on the launch
        stream, after `warm` untimed calls."""
        torch = self.torch
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        a.record(self.stream)
        for i in range(n):
            fn(i)
        b.record(self.stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e-3

    def per_call(self, fn, n):
        """Per-call durations (seconds), each call between its own events."""
        torch = self.torch
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for i, (a, b) in enumerate(evs):
            a.record(self.stream)
            fn(i)
            b.record(self.stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e-3 for a, b in evs]

    def stages(self, n):
        """Stage timings: kernel generation, the generating function (Cauchy
        kernel alone) and one convolution launch."""
        t_gen = self.timed(self.kernel_gen, n)
        t_cauchy = self.timed(self.cauchy, n)
        self.step(0)    # leaves this layer's spectrum (with D) in the workspace
        t_conv = self.timed(self.conv, n)
        return t_gen, t_cauchy, t_conv

    def close(self):
        self.plan.close()


def config_figures(wb, steps, warmup):
    """The per-workload entry of the ``configs`` map."""
    w = wb.w
    F1, Q2 = algorithmic_counts(w)
    for i in range(warmup):
        wb.step(i)
    wb.torch.cuda.synchronize()
    t_fwd = wb.timed(wb.step, steps, warm=0)
    per = wb.per_call(wb.step, steps)
    t_gen, t_cauchy, t_conv = wb.stages(steps)
    samples = w.batch * w.H * w.L
    s1_kernel_t = t_gen if fused_stage1(w.L) else t_cauchy
    return {
        "H": w.H, "N": w.N, "L": w.L, "batch": w.batch, "init": w.init,
        "forward_us": t_fwd * 1e6,
        "forward_us_median": statistics.median(per) * 1e6,
        "forward_us_min": min(per) * 1e6,
        "samples_per_s": samples / t_fwd,
        "stage1_us": t_gen * 1e6,
        "stage1_frac_fp32_peak": F1 / t_gen / 1e12 / FP32_PEAK_TFLOPS,
        "stage1_kernel": stage1_kernel_name(w.L),
        "stage1_kernel_us": s1_kernel_t * 1e6,
        "stage1_kernel_frac_fp32_peak": F1 / s1_kernel_t / 1e12 / FP32_PEAK_TFLOPS,
        "cauchy_algorithmic_flops": F1,
        "conv_kernels": conv_kernel_names(w.L),
        "conv_us": t_conv * 1e6,
        "conv_gbs": Q2 / t_conv / 1e9,
        "conv_frac_hbm": Q2 / t_conv / 1e9 / HBM_PEAK_GBS,
        "conv_algorithmic_bytes": Q2,
        "stage2_samples_per_s": samples / t_conv,
    }, (t_fwd, per, t_gen, t_cauchy, t_conv)


def secondary_legs(wb, steps, dev):
    """The (f) rows on the headline workload: recurrent view, zero-order hold,
    block and backward pass, each timed with HIP events on the launch stream."""
    s4, torch, w = wb.s4, wb.torch, wb.w
    p, P = wb.params, wb.P
    samples = w.batch * w.H * w.L
    out = {}
    flops_step, decode_bytes = recurrent_counts(w)
    s4.recurrent_prepare(wb.plan, p["lam"], P, p["Q"], p["B"], p["C"], p["dt"], wb.ws, wb.stream)
    state = torch.zeros((w.batch, w.H, w.N, 2), dtype=torch.float32, device=dev)
    scan = lambda i: s4.recurrent_scan(wb.plan, p["D"], wb.us[i % wb.nsets], state,
                                       wb.ys[i % wb.nsets], wb.ws, wb.stream)
    t_one = wb.timed(scan, 1)
    n_scan = max(3, min(steps, int(0.5 / max(t_one, 1e-6))))
    t_scan = wb.timed(scan, n_scan)
    u1 = wb.us[0][..., :1].contiguous()
    y1 = torch.empty_like(u1)
    t_dec = wb.timed(lambda i: s4.recurrent_scan(wb.plan, p["D"], u1, state, y1, wb.ws,
                                                 wb.stream), 200)
    rec_tflops = flops_step * w.L / t_scan / 1e12
    log(f"[bench] recurrent scan {t_scan * 1e6:.1f} us ({samples / t_scan:.3g} samples/s, "
        f"{rec_tflops:.1f} TFLOP/s); decode step {t_dec * 1e6:.2f} us")
    out["recurrent"] = {
        "kernel": "recurrent_scan_kernel (O(N) bilinear DPLR step, carried state)",
        "scan_us": t_scan * 1e6, "scan_samples_per_s": samples / t_scan, "bound": "alu",
        "achieved": rec_tflops, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": rec_tflops / FP32_PEAK_TFLOPS, "algorithmic_flops_per_step": flops_step,
        "decode_step_us": t_dec * 1e6, "decode_bytes_per_step": decode_bytes,
        "decode_tokens_per_s": w.batch / t_dec,
    }
    # zero-order hold (diagonal): the Vandermonde kernel on the same poles
    zplan = s4.Plan(w.H, w.N, w.L, w.batch, diagonal=True, zoh=True, device=dev)
    zws = zplan.workspace()
    t_vd = wb.timed(lambda i: s4.kernel_gen(zplan, p["lam"], None, None, p["B"], p["C"], p["dt"],
                                            wb.K, zws, wb.stream), steps)
    f_vd = 7 * w.H * w.L * w.N      # per (h, k, n): one complex product and one add
    log(f"[bench] zoh kernel_gen {t_vd * 1e6:.1f} us ({f_vd / t_vd / 1e9:.0f} GFLOP/s)")
    out["zoh"] = {"kernel_gen_us": t_vd * 1e6, "gflops": f_vd / t_vd / 1e9,
                  "frac_fp32_peak": f_vd / t_vd / 1e12 / FP32_PEAK_TFLOPS,
                  "algorithmic_flops": f_vd,
                  "note": "Vandermonde kernel plus the spectrum of K padded to 2L"}
    zplan.close()
    del zws
    # the block around the layer: layer norm, the layer, GLU projection
    from synth import make_block_params
    import numpy as np
    bp = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
          for k, v in make_block_params(w.H, seed=1).items()}
    bplan = s4.Plan(w.H, w.N, w.L, w.batch, diagonal=w.diagonal, device=dev, block=True)
    bws = bplan.workspace()
    t_blk = wb.timed(lambda i: s4.block_forward(
        bplan, wb.us[i % wb.nsets], bp["gamma"], bp["beta"], p["lam"], P, p["Q"], p["B"], p["C"],
        p["dt"], p["D"], bp["W"], bp["bias"], wb.ys[i % wb.nsets], bws, wb.stream), steps)
    f_proj = 2 * (2 * w.H) * w.H * w.batch * w.L        # the projection GEMM
    log(f"[bench] block forward {t_blk * 1e6:.1f} us ({samples / t_blk:.3g} samples/s)")
    out["block"] = {"us": t_blk * 1e6, "samples_per_s": samples / t_blk,
                    "projection_flops": f_proj,
                    "note": "layer norm + layer + GLU projection with residual (bf16 MFMA on "
                            "hi/lo split operands, fp32 accumulation)"}
    bplan.close()
    del bws
    # the backward pass: conv_bwd and kernel_gen_bwd
    q_bwd, f_bwd = backward_counts(w)
    dy, du = wb.ys[1 % wb.nsets], wb.ys[2 % wb.nsets]
    dK = torch.empty((w.H, w.L), dtype=torch.float32, device=dev)
    dD = torch.empty((w.H,), dtype=torch.float32, device=dev)
    grads = {k: torch.empty((w.H, w.N, 2), dtype=torch.float32, device=dev)
             for k in ("lam", "P", "B", "C")}
    ddt = torch.empty((w.H,), dtype=torch.float32, device=dev)
    t_cb = wb.timed(lambda i: s4.conv_bwd(wb.plan, wb.us[i % wb.nsets], wb.K, p["D"], dy, du, dK,
                                          dD, wb.ws, wb.stream), steps)
    t_kb = wb.timed(lambda i: s4.kernel_gen_bwd(
        wb.plan, p["lam"], P, p["Q"], p["B"], p["C"], p["dt"], dK, grads["lam"],
        None if w.diagonal else grads["P"], None, grads["B"], grads["C"], ddt, wb.ws,
        wb.stream), steps)
    log(f"[bench] conv_bwd {t_cb * 1e6:.1f} us ({q_bwd / t_cb / 1e9:.0f} GB/s), "
        f"kernel_gen_bwd {t_kb * 1e6:.1f} us ({f_bwd / t_kb / 1e9:.0f} GFLOP/s)")
    out["backward"] = {
        "conv_bwd_us": t_cb * 1e6, "conv_bwd_gbs": q_bwd / t_cb / 1e9,
        "conv_bwd_frac_hbm": q_bwd / t_cb / 1e9 / HBM_PEAK_GBS,
        "conv_bwd_algorithmic_bytes": q_bwd,
        "kernel_gen_bwd_us": t_kb * 1e6, "kernel_gen_bwd_gflops": f_bwd / t_kb / 1e9,
        "kernel_gen_bwd_frac_fp32_peak": f_bwd / t_kb / 1e12 / FP32_PEAK_TFLOPS,
        "kernel_gen_bwd_algorithmic_flops": f_bwd,
        "samples_per_s": samples / (t_cb + t_kb),
    }
    return out


def roofline(w, t_gen, t_cauchy, t_conv):
    """Roofline of the dominant kernel of the forward step, with the other
    stage beside it.  Stage 1 (the Cauchy sums) is bound by fp32 VALU
    arithmetic; the convolution nominally by HBM bandwidth.  The dominant
    kernel is the single kernel with the largest share of the step: the
    Cauchy kernel where the convolution is split over three four-step
    kernels (L >= 32768), else the slower of the two stages."""
    F1, Q2 = algorithmic_counts(w)
    traffic = read_traffic(w.name)
    s1_name = stage1_kernel_name(w.L)
    s1_t = t_gen if fused_stage1(w.L) else t_cauchy
    conv_names = conv_kernel_names(w.L)
    conv_traffic = None
    if all(k in traffic for k in conv_names):
        conv_traffic = sum(traffic[k] for k in conv_names)
    s1 = {"kernel": s1_name, "bound": "alu", "achieved": F1 / s1_t / 1e12,
          "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": F1 / s1_t / 1e12 / FP32_PEAK_TFLOPS,
          "traffic": traffic.get(s1_name), "algorithmic_flops_per_launch": F1,
          "launch_us": s1_t * 1e6,
          "stage1_us": t_gen * 1e6, "stage1_frac": F1 / t_gen / 1e12 / FP32_PEAK_TFLOPS}
    if w.L >= 32768:
        s1["note"] = ("launch_us times the generating-function entry point (cauchy_kernel, "
                      "HIP events). The forward pass runs the same sums in cauchy_half_kernel, "
                      "which also writes the half-length spectrum and the even spectrum bins "
                      "and has no entry point of its own; rocprofv3 averages of both kernels "
                      "are in profiles/<workload>_forward_kernel_trace.md")
    cv = {"kernel": " + ".join(conv_names), "bound": "hbm", "achieved": Q2 / t_conv / 1e9,
          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": Q2 / t_conv / 1e9 / HBM_PEAK_GBS,
          "traffic": conv_traffic, "algorithmic_bytes_per_launch": Q2,
          "launch_us": t_conv * 1e6,
          "valu_frac_fp32_peak": stage2_flops(w) / t_conv / 1e12 / FP32_PEAK_TFLOPS}
    if w.L >= 32768 or s1_t >= t_conv:
        main, other, other_key = s1, cv, "conv"
    else:
        main, other, other_key = cv, s1, "stage1_kernel"
    out = dict(main)
    out[other_key] = other
    return out


# ---------------------------------------------------------------------------
# rocprofv3 summaries
# ---------------------------------------------------------------------------

def _find_csv(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[-1]


def _short_name(name: str) -> str:
    """Kernel name without template arguments, parameters or launch suffix."""
    n = name.split("(")[0]
    n = n.split("<")[0]
    n = n.replace("void ", "").strip()
    return n.split("::")[-1]


def summarize_trace(d, label, command, by_grid=True):
    """Markdown table of per-kernel launch durations from a rocprofv3
    --kernel-trace run (kernel_trace.csv: end minus start per dispatch), one
    row per kernel and grid size (the same kernel serves launches of
    different sizes, e.g. the four-step kernels in stage 1 and in the
    convolution)."""
    path = _find_csv(d, "kernel_trace.csv")
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            key = _short_name(r["Kernel_Name"])
            if by_grid and "Grid_Size_X" in r:
                key += f" (grid {r['Grid_Size_X']}x{r.get('Grid_Size_Y', '1')})"
            per.setdefault(key, []).append(dur)
    total = sum(sum(v) for v in per.values())
    rows = sorted(per.items(), key=lambda kv: -sum(kv[1]))
    out = [f"# Kernel time per launch: {label}", "", "Command (run from the repository root):",
           "", "```", command, "```", "",
           "Source: `kernel_trace.csv` of rocprofv3 `--kernel-trace --stats`, durations are end "
           "minus start per dispatch, summarized by `python bench.py --summarize-trace`.", "",
           "| kernel | calls | average (us) | median (us) | min (us) | max (us) | share of GPU time |",
           "|---|---|---|---|---|---|---|"]
    for k, v in rows:
        out.append(f"| {k} | {len(v)} | {statistics.mean(v):.2f} | {statistics.median(v):.2f} | "
                   f"{min(v):.2f} | {max(v):.2f} | {100 * sum(v) / total:.1f}% |")
    return "\n".join(out) + "\n"


def _counter_rows(d):
    path = _find_csv(d, "counter_collection.csv")
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_counters(fetch_dir, write_dir, workload, commands):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the --counters launch
    sequence, scaled by what the same counters read for a plain 1 GiB copy:
    bytes per launch of each kernel, the median over its last five dispatches
    (the profiled calls; earlier dispatches of the same kernel belong to the
    set-up forward pass)."""
    out = {"workload": workload, "kernel_source_sha": kernel_source_hash(), "kernels": {},
           "commands": commands}
    vals = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for r in _counter_rows(d):
            if r.get("Counter_Name") != counter:
                continue
            name = _short_name(r["Kernel_Name"])
            key = (name, int(r.get("Dispatch_Id", r.get("Correlation_Id", 0))))
            vals.setdefault(counter, {}).setdefault(key, 0.0)
            vals[counter][key] += float(r["Counter_Value"])
    def per_kernel(counter):
        by = {}
        for (name, disp), v in sorted(vals[counter].items(), key=lambda kv: kv[0][1]):
            by.setdefault(name, []).append(v)
        return by
    fetch, write = per_kernel("FETCH_SIZE"), per_kernel("WRITE_SIZE")
    copy_bytes = 1 << 30
    copy_names = [k for k in fetch if "copy" in k.lower() or "elementwise" in k.lower()]
    # the calibration copy is the largest dispatch among the copy kernels
    cf = max((v for k in copy_names for v in fetch[k]), default=None)
    cw = max((v for k in copy_names for v in write.get(k, [])), default=None)
    if not cf or not cw:
        raise SystemExit("no calibration copy found in the counter runs")
    fscale, wscale = copy_bytes / (1024 * cf), copy_bytes / (1024 * cw)
    out["calibration"] = {"copy_bytes": copy_bytes, "copy_fetch_size_kib": cf,
                          "copy_write_size_kib": cw, "fetch_scale": fscale, "write_scale": wscale}
    names = ["cauchy_kernel", "kgen_wave_kernel", "conv_pair1024_kernel", "conv_wave_kernel",
             "conv_rows_kernel", "conv_kernel", "big_cols_fwd_kernel", "big_rows_pair_kernel",
             "big_cols_inv_kernel"]
    for k in names:
        if k in fetch and k in write:
            fk = statistics.median(fetch[k][-5:])
            wk = statistics.median(write[k][-5:])
            out["kernels"][k] = {"fetch_size_kib": fk, "write_size_kib": wk,
                                 "bytes_per_launch": fscale * 1024 * fk + wscale * 1024 * wk}
    out["formula"] = ("bytes = fetch_scale * 1024 * FETCH_SIZE + write_scale * 1024 * WRITE_SIZE "
                      "(KiB per dispatch, median over the kernel's profiled dispatches); scales "
                      "from a plain 1 GiB device copy in the same run")
    return out


SQ_COUNTERS = ("SQ_INSTS_VALU SQ_INSTS_LDS SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES "
               "SQ_WAIT_INST_LDS SQ_ACTIVE_INST_VALU SQ_WAIT_ANY GRBM_GUI_ACTIVE")


def summarize_sq(d, label, command):
    """Markdown table of the shader-sequencer counters of a --counters run
    (SQ_COUNTERS in one pass): per kernel, its last dispatch.  VALU issue is
    SQ_INSTS_VALU (wave instructions, all CUs) per CU per cycle, the cycles
    being GRBM_GUI_ACTIVE over the 8 XCDs; the wait shares are SQ_WAIT_ANY and
    SQ_WAIT_INST_LDS over SQ_WAVE_CYCLES."""
    per, meta = {}, {}
    for r in _counter_rows(d):
        key = (_short_name(r["Kernel_Name"]), int(r.get("Dispatch_Id", 0)))
        per.setdefault(key, {}).setdefault(r["Counter_Name"], 0.0)
        per[key][r["Counter_Name"]] += float(r["Counter_Value"])
        meta[key] = r
    last = {}   # by kernel and grid: one kernel serves launches of several sizes
    for key in sorted(per, key=lambda k: k[1]):
        last[(key[0], meta[key].get("Grid_Size", ""))] = key
    out = [f"# Shader-sequencer counters: {label}", "", "Command (run from the repository root):",
           "", "```", command, "```", "",
           "Source: `counter_collection.csv` of one rocprofv3 `--pmc` pass, the last dispatch of "
           "each kernel, summarized by `python bench.py --summarize-sq`.  VALU issue = "
           "SQ_INSTS_VALU / (256 CUs x GRBM_GUI_ACTIVE / 8); wait shares = SQ_WAIT_ANY and "
           "SQ_WAIT_INST_LDS over SQ_WAVE_CYCLES.", "",
           "| kernel | grid | workgroup | arch VGPRs | scratch (B) | duration (us) | VALU instr "
           "| VALU issue per CU-cycle | LDS instr | wait any | wait LDS |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    for (name, _), key in last.items():
        v, r = per[key], meta[key]
        cycles = v.get("GRBM_GUI_ACTIVE", 0.0) / 8
        wc = max(1.0, v.get("SQ_WAVE_CYCLES", 0.0))
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        issue = v.get("SQ_INSTS_VALU", 0.0) / (256 * cycles) if cycles else 0.0
        out.append(f"| {name} | {r.get('Grid_Size', '')} | {r.get('Workgroup_Size', '')} | "
                   f"{r.get('VGPR_Count', '')} | {r.get('Scratch_Size', '')} | {dur:.1f} | "
                   f"{v.get('SQ_INSTS_VALU', 0.0):.3g} | {issue:.2f} | "
                   f"{v.get('SQ_INSTS_LDS', 0.0):.3g} | {v.get('SQ_WAIT_ANY', 0.0) / wc:.2f} | "
                   f"{v.get('SQ_WAIT_INST_LDS', 0.0) / wc:.2f} |")
    return "\n".join(out) + "\n"


def counters_sequence(args):
    """The fixed launch sequence of a counter run: one forward pass (set-up),
    five generating-function calls, five convolution launches, then a plain
    1 GiB device copy for the counters' calibration."""
    import torch

    import structured_state_space_dplr_amd as s4
    from synth import WORKLOADS
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wb = Workbench(s4, torch, WORKLOADS[args.workload], dev)
    wb.step(0)
    for i in range(5):
        wb.cauchy(i)
    for i in range(5):
        wb.conv(i)
    torch.cuda.synchronize()
    wb.close()
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] counter sequence done: {args.workload}")
    return 0


# ---------------------------------------------------------------------------

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE,
                    help="headline workload: tiny | mid | long | s4d_lin | waveform "
                         f"(default: {HEADLINE}, the largest)")
    ap.add_argument("--configs", default="all",
                    help="workloads of the configs map: all | none | comma-separated names")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the recurrent, ZOH, block and backward legs")
    ap.add_argument("--counters", action="store_true",
                    help="run only the counter-collection launch sequence")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-sq", metavar="DIR")
    ap.add_argument("--label", default="")
    ap.add_argument("--command", default="")
    ap.add_argument("--out", default="")
    args = ap.parse_args()

    if args.summarize_trace:
        text = summarize_trace(args.summarize_trace, args.label or args.workload, args.command)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text)
        else:
            sys.stdout.write(text)
        return 0
    if args.summarize_sq:
        text = summarize_sq(args.summarize_sq, args.label or args.workload, args.command)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text)
        else:
            sys.stdout.write(text)
        return 0
    if args.summarize_counters:
        cmds = [c for c in args.command.split(" ;; ") if c]
        res = summarize_counters(*args.summarize_counters, args.workload, cmds)
        text = json.dumps(res, indent=1)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text + "\n")
        else:
            print(text)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported: the channels shard across GPUs with no exchange, so the figure of "
              "interest is the one-GPU throughput at the full workload shape.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import structured_state_space_dplr_amd as s4
    from synth import WORKLOADS

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    if args.counters:
        return counters_sequence(args)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS[args.workload]
    log(f"[bench] workload {w.describe()}; generating inputs")
    wb = Workbench(s4, torch, w, dev)
    log(f"[bench] {wb.nsets} buffer sets of {wb.set_mib:.1f} MiB; warmup {args.warmup}")
    for i in range(args.warmup):
        wb.step(i)
    torch.cuda.synchronize()
    # ---- timed region: exactly K forward steps ---------------------------------
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(wb.stream)
    for i in range(args.steps):
        wb.step(i)
    ev1.record(wb.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms_events = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = 1e3 * wall / args.steps
    samples = w.batch * w.H * w.L
    value = samples / (wall / args.steps)
    log(f"[bench] forward: {ms_per_step * 1e3:.1f} us/step (events {fwd_ms_events * 1e3:.1f} us)")
    per = wb.per_call(wb.step, args.steps)
    log(f"[bench] forward per step: median {statistics.median(per) * 1e6:.1f} us, "
        f"minimum {min(per) * 1e6:.1f} us")
    # the first set's outputs, for the parity check against the oracle
    wb.step(0)
    torch.cuda.synchronize()
    K_gpu = wb.K.cpu().numpy().astype(np.float64)
    y_gpu = wb.ys[0].cpu().numpy().astype(np.float64)
    t_gen, t_cauchy, t_conv = wb.stages(args.steps)
    F1, Q2 = algorithmic_counts(w)
    log(f"[bench] kernel_gen {t_gen * 1e6:.1f} us ({F1 / t_gen / 1e9:.0f} GFLOP/s), "
        f"generating function {t_cauchy * 1e6:.1f} us ({F1 / t_cauchy / 1e9:.0f} GFLOP/s), "
        f"conv {t_conv * 1e6:.1f} us ({Q2 / t_conv / 1e9:.0f} GB/s)")
    secondary = {} if args.no_secondary else secondary_legs(wb, args.steps, dev)
    x_head = wb.x
    wb.close()
    del wb
    torch.cuda.empty_cache()

    # ---- every workload: the configs map -----------------------------------------
    names = (ALL_CONFIGS if args.configs == "all" else
             [] if args.configs == "none" else args.configs.split(","))
    configs = {}
    for name in names:
        cw = WORKLOADS[name]
        if name == w.name:
            configs[name] = {
                "H": w.H, "N": w.N, "L": w.L, "batch": w.batch, "init": w.init,
                "forward_us": fwd_ms_events * 1e3,
                "forward_us_median": statistics.median(per) * 1e6,
                "forward_us_min": min(per) * 1e6, "samples_per_s": samples / (fwd_ms_events * 1e-3),
                "stage1_us": t_gen * 1e6,
                "stage1_frac_fp32_peak": F1 / t_gen / 1e12 / FP32_PEAK_TFLOPS,
                "stage1_kernel": stage1_kernel_name(w.L),
                "stage1_kernel_us": (t_gen if fused_stage1(w.L) else t_cauchy) * 1e6,
                "stage1_kernel_frac_fp32_peak":
                    F1 / (t_gen if fused_stage1(w.L) else t_cauchy) / 1e12 / FP32_PEAK_TFLOPS,
                "cauchy_algorithmic_flops": F1, "conv_kernels": conv_kernel_names(w.L),
                "conv_us": t_conv * 1e6, "conv_gbs": Q2 / t_conv / 1e9,
                "conv_frac_hbm": Q2 / t_conv / 1e9 / HBM_PEAK_GBS, "conv_algorithmic_bytes": Q2,
                "stage2_samples_per_s": samples / t_conv}
            continue
        log(f"[bench] config {cw.describe()}")
        cb = Workbench(s4, torch, cw, dev)
        configs[name], _ = config_figures(cb, min(args.steps, 50), min(args.warmup, 5))
        c = configs[name]
        log(f"[bench]   forward {c['forward_us']:.1f} us ({c['samples_per_s']:.3g} samples/s); "
            f"stage 1 {c['stage1_us']:.1f} us (frac {c['stage1_frac_fp32_peak']:.3f}); "
            f"conv {c['conv_us']:.1f} us (frac {c['conv_frac_hbm']:.3f})")
        cb.close()
        del cb
        torch.cuda.empty_cache()

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
        "roofline": roofline(w, t_gen, t_cauchy, t_conv),
        "kernel_gen": {
            "us": t_gen * 1e6, "gflops": F1 / t_gen / 1e9,
            "frac_fp32_peak": F1 / t_gen / 1e12 / FP32_PEAK_TFLOPS, "algorithmic_flops": F1,
            "generating_function_us": t_cauchy * 1e6,
            "note": "stage 1 = pack + Cauchy/Woodbury + kernel spectrum; the generating "
                    "function is the Cauchy kernel alone; flops counted for the Cauchy sums",
        },
        "stage2_samples_per_s": samples / t_conv,
        "forward_us_events": fwd_ms_events * 1e3,
        "forward_us_median": statistics.median(per) * 1e6,
        "forward_us_min": min(per) * 1e6,
        "configs": configs,
        **secondary,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"[bench] CPU baseline: fp64 oracle, >= {args.cpu_seconds:.0f} s")
        cbl, parity = cpu_baseline(x_head, K_gpu, y_gpu, args.cpu_seconds)
        result["cpu_baseline"] = cbl
        result["parity"] = parity
        log(f"[bench] oracle {cbl['value']:.3g} samples/s; parity K {parity['K_max_rel_err']:.2e} "
            f"y {parity['y_max_rel_err']:.2e} (worst channel K "
            f"{parity['K_worst_channel_rel_err']:.2e}, y {parity['y_worst_channel_rel_err']:.2e})")
        cp = cpu_baseline_pool(x_head)
        result["cpu_baseline_pool"] = cp
        log(f"[bench] oracle on {cp['cores']} worker processes: {cp['value']:.3g} samples/s "
            f"({cp['cpu_model']})")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
