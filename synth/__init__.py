"""Seeded synthetic inputs for the S4 DPLR convolution-mode forward pass.

This module is shared by the GPU path's harness and by the oracle's tests.  It
holds none of the method's arithmetic: it only draws random numbers, reads the
stored initialization tables under ``synth/data`` and rounds everything to the
float32 arrays that the library receives.

Recipe (the five workloads and their draws):
  * Poles and input/low-rank vectors: the HiPPO-LegS DPLR initialization of
    "The S4 kernel, from scratch" (section 2), read from the stored tables
    (N = 16 and N = 64 poles, all kept), replicated to every channel; or the
    S4D-Lin initialization of the "S4" wiki page (section "S4D"):
    a_n = -1/2 + i*pi*n, with B_n = 1 and no low-rank term.
  * ``numpy.random.default_rng(seed)``, draws in this order: log(dt)[H]
    uniform on [log lo, log hi]; Re C[H,N] and Im C[H,N], each N(0, 1/2);
    D[H] ~ N(0, 1); then the input u[batch, H, L].
  * u is N(0,1), or +-1 with probability 1/2 each, or per row the sum of three
    sinusoids (amplitude U[0,1], frequency log-uniform on [1e-3, 0.5) cycles
    per sample, phase U[0, 2 pi)) plus 0.1 * N(0,1) noise.
  * Everything is generated in float64 and rounded to float32 once.
"""
from __future__ import annotations

import os
from dataclasses import dataclass

import numpy as np

_DATA = os.path.join(os.path.dirname(os.path.abspath(__file__)), "data")


@dataclass(frozen=True)
class Workload:
    name: str
    H: int
    N: int
    L: int
    batch: int
    init: str          # "hippo" (DPLR rank 1, Q = P) or "s4d_lin" (diagonal)
    dt_lo: float
    dt_hi: float
    u_kind: str        # "normal" | "binary" | "sines"

    @property
    def diagonal(self) -> bool:
        return self.init == "s4d_lin"

    def describe(self) -> str:
        return (f"{self.name}: H={self.H} N={self.N} L={self.L} batch={self.batch} "
                f"init={self.init} dt~logU[{self.dt_lo:g},{self.dt_hi:g}] u={self.u_kind}")


# The five workloads of the benchmark suite (sizes from the task's configuration
# list; unstated details follow the readings listed in the design notes).
WORKLOADS = {
    "tiny":     Workload("tiny",     4,   16, 256,   2,  "hippo",   1e-3, 1e-1, "normal"),
    "mid":      Workload("mid",      256, 64, 1024,  32, "hippo",   1e-3, 1e-1, "normal"),
    "long":     Workload("long",     128, 64, 16384, 8,  "hippo",   1e-4, 1e-1, "binary"),
    "s4d_lin":  Workload("s4d_lin",  512, 64, 4096,  16, "s4d_lin", 1e-3, 1e-1, "normal"),
    "waveform": Workload("waveform", 64,  64, 65536, 4,  "hippo",   1e-4, 1e-2, "sines"),
}


def load_dplr_table(N: int):
    """Stored HiPPO-LegS DPLR initialization for N poles: (Lambda, P, B) complex128.

    The table was written by ``synth/write_init_tables.py`` from the fp64
    oracle and is plain text: one pole per line, columns
    Re(Lambda) Im(Lambda) Re(P) Im(P) Re(B) Im(B).
    """
    path = os.path.join(_DATA, f"hippo_legs_dplr_N{N}.txt")
    if not os.path.exists(path):
        raise FileNotFoundError(f"no stored DPLR table for N={N}: {path}")
    a = np.loadtxt(path, dtype=np.float64, ndmin=2)
    if a.shape != (N, 6):
        raise ValueError(f"{path}: expected shape ({N}, 6), got {a.shape}")
    return a[:, 0] + 1j * a[:, 1], a[:, 2] + 1j * a[:, 3], a[:, 4] + 1j * a[:, 5]


def _ri(z):
    """complex -> (..., 2) float64 interleaved (re, im)."""
    z = np.asarray(z)
    return np.stack([z.real, z.imag], axis=-1).astype(np.float64)


def draw_u(rng, kind: str, batch: int, H: int, L: int) -> np.ndarray:
    if kind == "normal":
        return rng.standard_normal((batch, H, L))
    if kind == "binary":
        return rng.integers(0, 2, size=(batch, H, L)).astype(np.float64) * 2.0 - 1.0
    if kind == "sines":
        amp = rng.uniform(0.0, 1.0, size=(batch, H, 3))
        freq = np.exp(rng.uniform(np.log(1e-3), np.log(0.5), size=(batch, H, 3)))
        phase = rng.uniform(0.0, 2.0 * np.pi, size=(batch, H, 3))
        noise = rng.standard_normal((batch, H, L))
        t = np.arange(L, dtype=np.float64)
        u = 0.1 * noise
        for j in range(3):
            u += amp[:, :, j, None] * np.sin(2.0 * np.pi * freq[:, :, j, None] * t
                                             + phase[:, :, j, None])
        return u
    raise ValueError(f"unknown u kind {kind!r}")


def make_inputs(workload, seed: int = 0, batch: int | None = None, H: int | None = None,
                L: int | None = None):
    """float32 inputs for one workload (a name from WORKLOADS or a Workload).

    ``batch``, ``H`` and ``L`` may override the workload's sizes (same recipe,
    smaller or larger problem).  Returns a dict with keys lam, P, Q, B, C
    ([H, N, 2] float32; P and Q None for the diagonal initialization, Q None
    meaning Q = P), dt, D ([H] float32), u ([batch, H, L] float32), and the
    workload itself under "workload".
    """
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    H = w.H if H is None else H
    L = w.L if L is None else L
    batch = w.batch if batch is None else batch
    N = w.N
    rng = np.random.default_rng(seed)
    log_dt = rng.uniform(np.log(w.dt_lo), np.log(w.dt_hi), size=H)
    C = rng.normal(0.0, np.sqrt(0.5), size=(H, N)) + 1j * rng.normal(0.0, np.sqrt(0.5), size=(H, N))
    D = rng.standard_normal(H)
    u = draw_u(rng, w.u_kind, batch, H, L)
    if w.init == "hippo":
        lam1, P1, B1 = load_dplr_table(N)
        lam = np.broadcast_to(lam1, (H, N))
        P = np.broadcast_to(P1, (H, N))
        B = np.broadcast_to(B1, (H, N))
    elif w.init == "s4d_lin":
        n = np.arange(N, dtype=np.float64)
        lam = np.broadcast_to(-0.5 + 1j * np.pi * n, (H, N))
        P = None
        B = np.ones((H, N), dtype=np.complex128)
    else:
        raise ValueError(w.init)
    f32 = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.float32)
    return {
        "lam": f32(_ri(lam)), "P": f32(None if P is None else _ri(P)), "Q": None,
        "B": f32(_ri(B)), "C": f32(_ri(C)), "dt": f32(np.exp(log_dt)), "D": f32(D),
        "u": f32(u), "workload": w,
    }


def make_generic_inputs(H: int, N: int, L: int, batch: int, seed: int = 0,
                        diagonal: bool = False, distinct_q: bool = False,
                        dt_lo: float = 1e-3, dt_hi: float = 1e-1, rank: int = 1):
    """Per-channel random DPLR parameters (not an initialization from the
    pages) for robustness cases: Re(Lambda) in -[0.05, 1], Im(Lambda) in
    [-40, 40], P, B, C complex Gaussian drawn independently, so B is not a
    multiple of P; with ``distinct_q`` an independent Q of modest size.
    With ``rank`` r > 1, P (and Q) hold r vectors of N: shape [H, r, N, 2].

    Draw order: Lambda re, Lambda im, P, B, C, Q (if distinct), log dt, D, u.
    """
    rng = np.random.default_rng(seed)
    cn = lambda *s: rng.normal(0.0, np.sqrt(0.5), size=s) + 1j * rng.normal(0.0, np.sqrt(0.5), size=s)
    lam = -rng.uniform(0.05, 1.0, size=(H, N)) + 1j * rng.uniform(-40.0, 40.0, size=(H, N))
    lr = (H, N) if rank == 1 else (H, rank, N)
    P = cn(*lr)
    B = cn(H, N)
    C = cn(H, N)
    Q = 0.3 * cn(*lr) if distinct_q else None
    log_dt = rng.uniform(np.log(dt_lo), np.log(dt_hi), size=H)
    D = rng.standard_normal(H)
    u = rng.standard_normal((batch, H, L))
    f32 = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.float32)
    return {
        "lam": f32(_ri(lam)), "P": None if diagonal else f32(_ri(P)),
        "Q": None if (diagonal or Q is None) else f32(_ri(Q)),
        "B": f32(_ri(B)), "C": f32(_ri(C)), "dt": f32(np.exp(log_dt)), "D": f32(D),
        "u": f32(u), "workload": None,
    }


def make_block_params(H: int, seed: int = 1):
    """Random-initialized parameters of the block around the layer (pre-norm,
    GLU-gated projection): LayerNorm gain gamma = 1 + 0.1 N(0,1) and shift
    beta = 0.1 N(0,1) per channel, projection W (2H x H) with N(0, 1/H)
    entries (rows [0, H): the value half, rows [H, 2H): the gate half) and bias
    0.1 N(0,1) (2H).  Draw order: gamma, beta, W, bias.  fp32."""
    rng = np.random.default_rng(seed)
    gamma = 1.0 + 0.1 * rng.standard_normal(H)
    beta = 0.1 * rng.standard_normal(H)
    W = rng.standard_normal((2 * H, H)) / np.sqrt(H)
    bias = 0.1 * rng.standard_normal(2 * H)
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return {"gamma": f32(gamma), "beta": f32(beta), "W": f32(W), "bias": f32(bias)}
