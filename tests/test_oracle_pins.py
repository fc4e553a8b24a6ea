"""Pins for the fp64 oracle: values and identities fixed by the pages and by
mathematics, chosen so that a dropped term, a wrong sign or index, or a
transposed operand anywhere in ``oracle/`` fails at least one of them.

Pages: "The S4 kernel, from scratch" ([scratch]); "S4" wiki ([wiki]);
"Structured state-space sequence model and S4" ([glossary]).
"""
import os

import numpy as np
import pytest

import oracle as o
from synth import load_dplr_table, make_generic_inputs, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split()
            vals[k] = float(v)
    return vals


def _cn(rng, *shape):
    return rng.normal(size=shape) + 1j * rng.normal(size=shape)


# --- P1: the worked example of [glossary] "Follow one input through memory" --

def test_worked_example_zoh_values():
    g = _golden("worked_example_zoh.txt")
    Abar, Bbar = o.discretize_zoh_scalar(g["a"], g["b"], g["dt"])
    assert abs(Abar - g["Abar"]) < 1e-10
    assert abs(Bbar - g["Bbar"]) < 1e-10


def test_worked_example_recurrence_and_convolution():
    g = _golden("worked_example_zoh.txt")
    Abar, Bbar = o.discretize_zoh_scalar(g["a"], g["b"], g["dt"])
    A1, B1, C1 = np.array([[Abar]]), np.array([Bbar]), np.array([g["c"]])
    u = np.array([1.0, 0.0])
    y_rec = o.recurrence(A1, B1, C1, 0.0, u)
    assert abs(y_rec[0] - g["h1"]) < 1e-10 and abs(y_rec[1] - g["h2"]) < 1e-10
    K = o.kernel_truncated(A1, B1, C1, 2)
    assert abs(K[0] - g["k0"]) < 1e-10 and abs(K[1] - g["k1"]) < 1e-10
    y_conv = o.conv_direct(u, K, 0.0)
    np.testing.assert_allclose(y_conv, [g["h1"], g["h2"]], atol=1e-10)
    np.testing.assert_allclose(o.conv_fft(u, K, 0.0), [g["h1"], g["h2"]], atol=1e-10)


def test_zoh_limit_at_zero_pole():
    # a -> 0: exp(dt a) -> 1 and (exp(dt a) - 1)/a * b -> dt b.
    Abar, Bbar = o.discretize_zoh_scalar(0.0, 3.0, 0.25)
    assert Abar == 1.0 and Bbar == 0.75
    # near a = 0 the series b (dt + a dt^2 / 2 + ...) holds
    A2, B2 = o.discretize_zoh_scalar(-1e-9, 3.0, 0.25)
    assert abs(B2 - 3.0 * (0.25 - 1e-9 * 0.25 ** 2 / 2)) < 1e-15


# --- P2: scalar bilinear closed form ---------------------------------------

@pytest.mark.parametrize("L", [2, 4, 16, 256])
def test_scalar_bilinear_closed_form(L):
    # Lambda = -1, B = C = 1, dt = 1, no low-rank term:
    # A-bar = 1/3, B-bar = 2/3, K-hat(z) = 2/(3 - z), K_k = (2/3) 3^-k / (1 - 3^-L).
    Abar, Bbar = o.discretize_bilinear(np.array([[-1.0]]), np.array([1.0]), 1.0)
    assert abs(Abar[0, 0] - 1.0 / 3.0) < 1e-15 and abs(Bbar[0] - 2.0 / 3.0) < 1e-15
    lam, z0, one = np.array([-1.0 + 0j]), np.array([0j]), np.array([1.0 + 0j])
    k = np.arange(L)
    ref = (2.0 / 3.0) * 3.0 ** (-k) / (1.0 - 3.0 ** (-L))
    Kh = o.generating_function(lam, z0, z0, one, one, 1.0, L)
    z = np.exp(-2j * np.pi * k / L)
    np.testing.assert_allclose(Kh, 2.0 / (3.0 - z), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(o.kernel_cauchy(lam, z0, z0, one, one, 1.0, L), ref, rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(o.kernel_aliased_dense(Abar, Bbar, one, L), ref, rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(o.kernel_truncated(Abar, Bbar, one, L), (2.0 / 3.0) * 3.0 ** (-k), rtol=1e-12, atol=1e-16)


# --- P3: rank-1 Woodbury with N = 1 equals a shifted diagonal pole ----------

def test_scalar_woodbury_equals_shifted_pole():
    rng = np.random.default_rng(1)
    for _ in range(5):
        lam = np.array([-rng.uniform(0.1, 2.0) + 1j * rng.uniform(-5, 5)])
        p, b, c = _cn(rng, 1), _cn(rng, 1), _cn(rng, 1)
        dt, L = rng.uniform(0.01, 0.5), 64
        K_dplr = o.kernel_cauchy(lam, p, p, b, c, dt, L)
        a = lam - np.abs(p) ** 2
        K_diag = o.kernel_cauchy(a, 0 * p, 0 * p, b, c, dt, L)
        np.testing.assert_allclose(K_dplr, K_diag, rtol=1e-11, atol=1e-13)
        # closed form of the scalar bilinear system, summed over all periods
        Ab = (1 + dt * a[0] / 2) / (1 - dt * a[0] / 2)
        Bb = dt * b[0] / (1 - dt * a[0] / 2)
        k = np.arange(L)
        ref = (c[0] * Bb * Ab ** k / (1 - Ab ** L)).real
        np.testing.assert_allclose(K_dplr, ref, rtol=1e-10, atol=1e-12)


# --- Woodbury/Cauchy sums against a direct linear solve of the resolvent ----

def test_generating_function_matches_resolvent_solve():
    rng = np.random.default_rng(2)
    N, L, dt = 6, 32, 0.07
    lam = -rng.uniform(0.1, 1.0, N) + 1j * rng.uniform(-10, 10, N)
    P, Q, B, C = _cn(rng, N), 0.5 * _cn(rng, N), _cn(rng, N), _cn(rng, N)
    Kh = o.generating_function(lam, P, Q, B, C, dt, L)
    A = np.diag(lam) - np.outer(P, Q.conj())      # A = Lambda - P Q^*
    for l in range(L):
        if l == L // 2:
            continue
        z = np.exp(-2j * np.pi * l / L)
        g = (2 / dt) * (1 - z) / (1 + z)
        ref = (2 / (1 + z)) * (C @ np.linalg.solve(g * np.eye(N) - A, B))
        assert abs(Kh[l] - ref) <= 1e-11 * max(1.0, abs(ref))


def test_generating_function_is_power_series_of_markov_parameters():
    # K-hat(z) = sum_k (C A-bar^k B-bar) z^k for the bilinear system, summed
    # until the terms have decayed (Delta large enough for fast decay).
    rng = np.random.default_rng(3)
    N, L, dt = 5, 16, 0.5
    lam = -rng.uniform(0.5, 1.5, N) + 1j * rng.uniform(-3, 3, N)
    P, B, C = 0.3 * _cn(rng, N), _cn(rng, N), _cn(rng, N)
    Kh = o.generating_function(lam, P, P, B, C, dt, L)
    Abar, Bbar = o.discretize_bilinear(o.dense_state_matrix(lam, P, P), B, dt)
    z = np.exp(-2j * np.pi * np.arange(L) / L)
    acc = np.zeros(L, complex)
    x = Bbar.copy()
    zk = np.ones(L, complex)
    for _ in range(4000):
        acc += (C @ x) * zk
        x = Abar @ x
        zk = zk * z
    assert np.abs(C @ x) < 1e-14
    np.testing.assert_allclose(Kh, acc, rtol=1e-10, atol=1e-12)


# --- P4: DC and Nyquist closed forms ---------------------------------------

@pytest.mark.parametrize("L", [8, 256, 1024])
def test_dc_and_nyquist_sums(L):
    lam, P, B = load_dplr_table(16)
    rng = np.random.default_rng(4)
    C = _cn(rng, 16)
    dt = 0.03
    K = o.kernel_cauchy(lam, P, P, B, C, dt, L)
    A = o.dense_state_matrix(lam, P, P)
    dc = (-C @ np.linalg.solve(A, B)).real           # K-hat at z = 1
    nyq = (dt / 2 * np.sum(C * B)).real                # K-hat at z = -1
    s = np.abs(K).sum()
    assert abs(K.sum() - dc) <= 1e-12 * s
    assert abs((K * (-1.0) ** np.arange(L)).sum() - nyq) <= 1e-12 * s


# --- P5 / P6: HiPPO-LegS -> NPLR -> DPLR invariants --------------------------

@pytest.mark.parametrize("N", [4, 16, 64])
def test_hippo_nplr_dplr_invariants(N):
    A, P, B, S = o.nplr_legs(N)
    # the normal part is normal: S S^T = S^T S, with diagonal -1/2 and a skew rest
    nS = np.linalg.norm(S)
    assert np.linalg.norm(S @ S.T - S.T @ S) <= 1e-12 * nS ** 2
    np.testing.assert_allclose(np.diag(S), -0.5, atol=1e-14)
    T = S + 0.5 * np.eye(N)
    assert np.abs(T + T.T).max() <= 1e-13
    lam, Pt, Bt, V = o.dplr_legs(N)
    assert np.linalg.norm(V.conj().T @ V - np.eye(N)) <= 1e-12
    Ad = o.dense_state_matrix(lam, Pt, Pt)
    assert np.linalg.norm(V @ Ad @ V.conj().T - A) <= 1e-13 * np.linalg.norm(A)
    np.testing.assert_allclose(lam.real, -0.5, atol=1e-13)
    assert np.all(np.diff(lam.imag) >= 0)
    assert np.abs(Pt.imag).max() <= 1e-12 and Pt.real.min() >= 0
    # B = sqrt(2) P holds for LegS before and after the change of basis
    np.testing.assert_allclose(B, np.sqrt(2) * P, rtol=1e-15)
    np.testing.assert_allclose(Bt, np.sqrt(2) * Pt, atol=1e-12 * np.abs(Bt).max())


def test_stored_tables_match_oracle():
    for N in (16, 64):
        lam, P, B = load_dplr_table(N)
        lam2, P2, B2, _ = o.dplr_legs(N)
        np.testing.assert_allclose(lam, lam2, atol=1e-12 * np.abs(lam2).max())
        np.testing.assert_allclose(P, P2, atol=1e-12 * np.abs(P2).max())
        np.testing.assert_allclose(B, B2, atol=1e-12 * np.abs(B2).max())


# --- P7: the Woodbury denominator stays away from zero when Q = P ----------

def test_woodbury_denominator_bound():
    lam, P, B = load_dplr_table(64)
    for dt in (1e-4, 1e-2, 1e-1):
        L = 4096
        l = np.arange(L)
        l = l[l != L // 2]
        z = np.exp(-2j * np.pi * l / L)
        g = (2 / dt) * (1 - z) / (1 + z)
        k11 = (1 / (g[:, None] - lam[None, :])) @ (np.conj(P) * P)
        assert np.abs(1 + k11).min() >= 1 - 1e-12


# --- P8: aliasing identity (Cauchy method == dense aliased definition) ------

@pytest.mark.parametrize("N,L,dt", [(16, 256, 1e-3), (16, 256, 1e-1), (64, 1024, 1e-2), (64, 512, 1e-4)])
def test_cauchy_equals_dense_aliased_hippo(N, L, dt):
    lam, P, B = load_dplr_table(N)
    C = _cn(np.random.default_rng(N + L), N) * np.sqrt(0.5)
    K1 = o.kernel_cauchy(lam, P, P, B, C, dt, L)
    Abar, Bbar = o.discretize_bilinear(o.dense_state_matrix(lam, P, P), B, dt)
    K2 = o.kernel_aliased_dense(Abar, Bbar, C, L)
    assert np.abs(K1 - K2).max() <= 1e-10 * np.abs(K2).max()


def test_cauchy_equals_dense_aliased_generic_distinct_q():
    x = make_generic_inputs(H=3, N=8, L=128, batch=1, seed=5, distinct_q=True)
    K1, _ = o.forward(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], x["D"], x["u"], method="cauchy")
    K2, _ = o.forward(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], x["D"], x["u"], method="dense")
    assert np.abs(K1 - K2).max() <= 1e-10 * np.abs(K2).max()


def test_aliased_kernel_is_sum_over_periods():
    # [scratch] section 4, "Aliasing": the kernel matches a dense system summed
    # over many periods (the page's tolerance: < 1e-4).
    lam, P, B = load_dplr_table(16)
    C = _cn(np.random.default_rng(7), 16) * np.sqrt(0.5)
    dt, L, periods = 1e-2, 128, 200
    K = o.kernel_cauchy(lam, P, P, B, C, dt, L)
    Abar, Bbar = o.discretize_bilinear(o.dense_state_matrix(lam, P, P), B, dt)
    Kt = o.kernel_truncated(Abar, Bbar, C, L * periods).reshape(periods, L).sum(0)
    assert np.abs(K - Kt).max() / np.abs(Kt).max() < 1e-4


# --- P9: decayed kernel equals the exact recurrence -------------------------

def test_decayed_kernel_matches_recurrence():
    lam, P, B = load_dplr_table(16)
    C = _cn(np.random.default_rng(8), 16) * np.sqrt(0.5)
    dt, L = 0.1, 1024
    Abar, Bbar = o.discretize_bilinear(o.dense_state_matrix(lam, P, P), B, dt)
    assert np.abs(np.linalg.eigvals(Abar)).max() ** L < 1e-8
    K = o.kernel_cauchy(lam, P, P, B, C, dt, L)
    Kt = o.kernel_truncated(Abar, Bbar, C, L)
    assert np.abs(K - Kt).max() / np.abs(Kt).max() < 1e-7      # page: ~1e-7
    u = np.random.default_rng(9).standard_normal(L)
    y_rec = o.recurrence(Abar, Bbar, C, 0.3, u)
    y_conv = o.conv_fft(u, K, 0.3)
    assert np.abs(y_rec - y_conv).max() / np.abs(y_rec).max() < 1e-7


# --- P10: diagonal (S4D) Vandermonde closed form ----------------------------

def test_s4d_lin_vandermonde_closed_form():
    x = make_inputs("s4d_lin", H=2, batch=1, L=4096)
    lam = x["lam"][..., 0].astype(np.float64) + 1j * x["lam"][..., 1]
    C = x["C"][..., 0].astype(np.float64) + 1j * x["C"][..., 1]
    Bv = x["B"][..., 0].astype(np.float64) + 1j * x["B"][..., 1]
    L = 4096
    K, _ = o.forward(x["lam"], None, None, x["B"], x["C"], x["dt"], x["D"], x["u"], diagonal=True)
    k = np.arange(L)
    for h in range(2):
        dt = float(x["dt"][h])
        Ab = (1 + dt * lam[h] / 2) / (1 - dt * lam[h] / 2)
        Bb = dt * Bv[h] / (1 - dt * lam[h] / 2)
        ref = ((C[h] * Bb / (1 - Ab ** L))[None, :] * Ab[None, :] ** k[:, None]).sum(1).real
        assert np.abs(K[h] - ref).max() <= 1e-11 * np.abs(ref).max()


# --- Recurrent view from a carried state -----------------------------------

def test_recurrence_from_state_scalar_closed_form():
    # zero input: x_t = a^(t+1) x0, so y_t = Re(c a^(t+1) x0) for every sequence
    a, b, c = 0.9 * np.exp(0.3j), 0.7 - 0.2j, 1.3 + 0.4j
    x0 = np.array([[1.0 - 2.0j], [0.5j], [-0.25 + 0.0j]])
    T = 12
    y, xT = o.recurrence(np.array([[a]]), np.array([b]), np.array([c]), 0.0,
                         np.zeros((3, T)), x0=x0, return_state=True)
    t = np.arange(T)
    ref = (c * a ** (t[None, :] + 1) * x0).real
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-15)
    np.testing.assert_allclose(xT, a ** T * x0, rtol=0, atol=1e-15)


def test_recurrence_from_state_superposition_and_explicit_state():
    # y(u, x0) = y(u, 0) + Re(C A-bar^(t+1) x0); x_T = A-bar^T x0 + sum_j A-bar^(T-1-j) B-bar u_j
    rng = np.random.default_rng(21)
    N, T = 4, 9
    lam = -rng.uniform(0.1, 1, N) + 1j * rng.uniform(-2, 2, N)
    P, B, C = 0.5 * _cn(rng, N), _cn(rng, N), _cn(rng, N)
    Abar, Bbar = o.discretize_bilinear(o.dense_state_matrix(lam, P, P), B, 0.3)
    u = rng.standard_normal((2, T))
    x0 = _cn(rng, 2, N)
    y, xT = o.recurrence(Abar, Bbar, C, 0.4, u, x0=x0, return_state=True)
    y0 = o.recurrence(Abar, Bbar, C, 0.4, u)
    for s in range(2):
        free = np.array([(C @ np.linalg.matrix_power(Abar, t + 1) @ x0[s]).real for t in range(T)])
        np.testing.assert_allclose(y[s], y0[s] + free, rtol=0, atol=1e-13 * np.abs(y[s]).max())
        ref = np.linalg.matrix_power(Abar, T) @ x0[s]
        for j in range(T):
            ref = ref + np.linalg.matrix_power(Abar, T - 1 - j) @ Bbar * u[s, j]
        np.testing.assert_allclose(xT[s], ref, rtol=0, atol=1e-13 * np.abs(ref).max())


@pytest.mark.parametrize("diagonal,distinct_q", [(False, False), (False, True), (True, False)])
def test_recurrent_forward_equals_truncated_convolution(diagonal, distinct_q):
    # every (batch, channel) sequence: zero-state response = causal convolution
    # with the truncated kernel C A-bar^k B-bar of that channel
    x = make_generic_inputs(H=3, N=4, L=16, batch=2, seed=5, diagonal=diagonal,
                            distinct_q=distinct_q)
    y, _ = o.recurrent_forward(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], x["D"], x["u"],
                               diagonal=diagonal)
    c = lambda a: a[..., 0].astype(np.float64) + 1j * a[..., 1]
    for h in range(3):
        P = np.zeros(4) if diagonal else c(x["P"][h])
        Q = P if (diagonal or x["Q"] is None) else c(x["Q"][h])
        Abar, Bbar = o.discretize_bilinear(o.dense_state_matrix(c(x["lam"][h]), P, Q),
                                           c(x["B"][h]), float(x["dt"][h]))
        Kt = o.kernel_truncated(Abar, Bbar, c(x["C"][h]), 16)
        for b in range(2):
            ref = o.conv_direct(x["u"][b, h], Kt, float(x["D"][h]))
            np.testing.assert_allclose(y[b, h], ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_recurrent_forward_split_equals_whole():
    x = make_generic_inputs(H=2, N=5, L=32, batch=3, seed=6)
    args = (x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], x["D"])
    y, xT = o.recurrent_forward(*args, x["u"])
    y1, x1 = o.recurrent_forward(*args, x["u"][..., :11])
    y2, x2 = o.recurrent_forward(*args, x["u"][..., 11:], x0=x1)
    np.testing.assert_allclose(np.concatenate([y1, y2], -1), y, rtol=0, atol=1e-13)
    np.testing.assert_allclose(x2, xT, rtol=0, atol=1e-13)


# --- P11 / P12: brute force on tiny inputs ----------------------------------

@pytest.mark.parametrize("N,L", [(1, 4), (2, 8), (4, 16), (3, 16)])
def test_recurrence_equals_convolution_bruteforce(N, L):
    rng = np.random.default_rng(10 + N)
    lam = -rng.uniform(0.1, 1, N) + 1j * rng.uniform(-2, 2, N)
    P, B, C = 0.5 * _cn(rng, N), _cn(rng, N), _cn(rng, N)
    dt, D = 0.2, rng.normal()
    Abar, Bbar = o.discretize_bilinear(o.dense_state_matrix(lam, P, P), B, dt)
    Kt = o.kernel_truncated(Abar, Bbar, C, L)
    for trial in range(3):
        u = rng.standard_normal(L)
        y1 = o.recurrence(Abar, Bbar, C, D, u)
        y2 = o.conv_direct(u, Kt, D)
        y3 = o.conv_fft(u, Kt, D)
        np.testing.assert_allclose(y1, y2, atol=1e-13 * np.abs(y1).max())
        np.testing.assert_allclose(y1, y3, atol=1e-13 * np.abs(y1).max())
    for t0 in range(L):             # unit impulses: the response is the shifted kernel
        u = np.zeros(L)
        u[t0] = 1.0
        y = o.recurrence(Abar, Bbar, C, D, u)
        ref = np.zeros(L)
        ref[t0:] = Kt[: L - t0]
        ref[t0] += D
        np.testing.assert_allclose(y, ref, atol=1e-13)


@pytest.mark.parametrize("L", [1, 2, 4, 8, 32, 128])
def test_fft_convolution_equals_direct(L):
    rng = np.random.default_rng(L)
    u, K, D = rng.standard_normal(L), rng.standard_normal(L), rng.normal()
    y = o.conv_fft(u, K, D)
    np.testing.assert_allclose(y, o.conv_direct(u, K, D), atol=1e-12 * max(1, np.abs(y).max()))
    for t in range(L):
        assert abs(o.conv_direct_at(u, K, D, t) - y[t]) < 1e-12 * max(1, np.abs(y).max())
    # causality: changing a later input does not change earlier outputs
    if L > 1:
        u2 = u.copy()
        u2[L // 2:] += 1.0
        np.testing.assert_allclose(o.conv_fft(u2, K, D)[: L // 2], y[: L // 2], atol=1e-12)
    # broadcasting over (batch, H) rows equals the per-row result
    U = rng.standard_normal((2, 3, L))
    Ks = rng.standard_normal((3, L))
    Ds = rng.standard_normal(3)
    Y = o.conv_fft(U, Ks[None], Ds[None, :, None])
    for b in range(2):
        for h in range(3):
            np.testing.assert_allclose(Y[b, h], o.conv_direct(U[b, h], Ks[h], Ds[h]), atol=1e-11)


# --- P13: discrete stability ------------------------------------------------

def test_discrete_poles_inside_unit_circle():
    for N in (16, 64):
        lam, P, B = load_dplr_table(N)
        for dt in (1e-4, 1e-2, 1e-1):
            Abar, _ = o.discretize_bilinear(o.dense_state_matrix(lam, P, P), B, dt)
            assert np.abs(np.linalg.eigvals(Abar)).max() < 1.0


def test_forward_tiny_cauchy_vs_dense():
    x = make_inputs("tiny")
    K1, y1 = o.forward(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], x["D"], x["u"], method="cauchy")
    K2, y2 = o.forward(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], x["D"], x["u"], method="dense")
    assert np.abs(K1 - K2).max() <= 1e-10 * np.abs(K2).max()
    assert np.abs(y1 - y2).max() <= 1e-10 * np.abs(y2).max()
    # y against the direct sum on every row
    for b in range(y1.shape[0]):
        for h in range(y1.shape[1]):
            yd = o.conv_direct(x["u"][b, h], K2[h], float(x["D"][h]))
            assert np.abs(yd - y1[b, h]).max() <= 1e-11 * np.abs(yd).max()


# --- Backward pass ------------------------------------------------------------

def test_conv_backward_adjoint_identities():
    # y is linear in u, and jointly linear in (K, D): for every u, K, D,
    # sum(dy * y) = sum(du * u) = sum(dK * K) + sum(dD * D)
    rng = np.random.default_rng(30)
    for (Bt, H, L) in [(2, 3, 1), (2, 3, 2), (3, 2, 17), (1, 4, 64)]:
        u, dy = rng.standard_normal((Bt, H, L)), rng.standard_normal((Bt, H, L))
        K, D = rng.standard_normal((H, L)), rng.standard_normal(H)
        y = np.array([[o.conv_direct(u[b, h], K[h], D[h]) for h in range(H)] for b in range(Bt)])
        du, dK, dD = o.conv_backward_direct(u, K, D, dy)
        s = np.sum(dy * y)
        assert abs(np.sum(du * u) - s) <= 1e-12 * (1 + abs(s))
        assert abs(np.sum(dK * K) + np.sum(dD * D) - s) <= 1e-12 * (1 + abs(s))


def test_conv_backward_impulses():
    # dy a unit impulse at t0 picks out the row of the Jacobian: du[t] = K[t0-t] (t <= t0)
    # plus D at t0; dK[j] = u[t0-j]; dD = u[t0]
    rng = np.random.default_rng(31)
    L = 9
    u, K, D = rng.standard_normal((1, 1, L)), rng.standard_normal((1, L)), rng.standard_normal(1)
    for t0 in range(L):
        dy = np.zeros((1, 1, L))
        dy[0, 0, t0] = 1.0
        du, dK, dD = o.conv_backward_direct(u, K, D, dy)
        ref = np.zeros(L)
        ref[: t0 + 1] = K[0, t0::-1]
        ref[t0] += D[0]
        np.testing.assert_allclose(du[0, 0], ref, atol=1e-15)
        refk = np.zeros(L)
        refk[: t0 + 1] = u[0, 0, t0::-1]
        np.testing.assert_allclose(dK[0], refk, atol=1e-15)
        assert dD[0] == u[0, 0, t0]


@pytest.mark.parametrize("L", [2, 8, 64, 256])
def test_conv_backward_fft_equals_direct(L):
    rng = np.random.default_rng(32)
    u, dy = rng.standard_normal((3, 2, L)), rng.standard_normal((3, 2, L))
    K, D = rng.standard_normal((2, L)), rng.standard_normal(2)
    a = o.conv_backward_direct(u, K, D, dy)
    b = o.conv_backward_fft(u, K, D, dy)
    for x, y in zip(a, b):
        np.testing.assert_allclose(y, x, rtol=0, atol=1e-12 * np.abs(x).max())


def _kernel_loss(x, dK, diagonal=False):
    K, _ = o.forward(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], np.zeros(len(x["dt"])),
                     np.zeros((1,) + dK.shape), method="dense", diagonal=diagonal)
    return float(np.sum(K * dK))


@pytest.mark.parametrize("diagonal,distinct_q", [(False, False), (False, True), (True, False)])
def test_kernel_backward_finite_differences(diagonal, distinct_q):
    # central differences of the dense aliased kernel, one real component at a time
    x = make_generic_inputs(H=2, N=3, L=8, batch=1, seed=33, diagonal=diagonal,
                            distinct_q=distinct_q)
    x = {k: (None if v is None or k == "workload" else np.asarray(v, np.float64))
         for k, v in x.items()}
    dK = np.random.default_rng(34).standard_normal((2, 8))
    g = o.kernel_backward_dense(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], dK,
                                diagonal=diagonal)
    names = ["lam", "B", "C", "dt"] + ([] if diagonal else ["P"] + (["Q"] if distinct_q else []))
    for name in names:
        flat = x[name].reshape(-1)
        for i in range(flat.size):
            e = 1e-6 * max(1.0, abs(flat[i]))
            xp = {k: (None if v is None else v.copy()) for k, v in x.items()}
            xm = {k: (None if v is None else v.copy()) for k, v in x.items()}
            xp[name].reshape(-1)[i] += e
            xm[name].reshape(-1)[i] -= e
            fd = (_kernel_loss(xp, dK, diagonal) - _kernel_loss(xm, dK, diagonal)) / (2 * e)
            an = g[name].reshape(-1)[i]
            assert abs(fd - an) <= 1e-5 * max(1.0, abs(an)), (name, i, fd, an)


def test_kernel_backward_scalar_closed_form():
    # N = 1, diagonal: K_k = Re(c m_k) with m_k = b-bar a-bar^k / (1 - a-bar^L), so
    # dloss/dRe(c) + i dloss/dIm(c) = sum_k dK_k conj(m_k), and the same with c and b swapped
    # through b-bar = dt b / (1 - dt lam / 2)
    lam, b, c, dt, L = -0.3 + 2.0j, 0.8 - 0.4j, 1.1 + 0.6j, 0.25, 16
    ab = (1 + dt * lam / 2) / (1 - dt * lam / 2)
    bb = dt * b / (1 - dt * lam / 2)
    k = np.arange(L)
    dK = np.random.default_rng(35).standard_normal((1, L))
    m = bb * ab ** k / (1 - ab ** L)
    ri = lambda z: np.array([[[z.real, z.imag]]])
    g = o.kernel_backward_dense(ri(lam), None, None, ri(b), ri(c), np.array([dt]), dK,
                                diagonal=True)
    gc = np.sum(dK[0] * np.conj(m))
    np.testing.assert_allclose(g["C"][0, 0], [gc.real, gc.imag], rtol=1e-12)
    gb = np.sum(dK[0] * np.conj(c * m / b))
    np.testing.assert_allclose(g["B"][0, 0], [gb.real, gb.imag], rtol=1e-12)


def test_kernel_backward_tied_q_is_sum_of_both_paths():
    x = make_generic_inputs(H=1, N=4, L=8, batch=1, seed=36)
    dK = np.random.default_rng(37).standard_normal((1, 8))
    tied = o.kernel_backward_dense(x["lam"], x["P"], None, x["B"], x["C"], x["dt"], dK)
    split = o.kernel_backward_dense(x["lam"], x["P"], x["P"], x["B"], x["C"], x["dt"], dK)
    np.testing.assert_allclose(tied["P"], split["P"] + split["Q"], rtol=1e-12, atol=1e-14)
    for k in ("lam", "B", "C", "dt"):
        np.testing.assert_allclose(tied[k], split[k], rtol=1e-12, atol=1e-14)


# --- Zero-order hold, diagonal: the Vandermonde kernel ---------------------------

def test_zoh_vandermonde_worked_example():
    g = _golden("worked_example_zoh.txt")
    K = o.kernel_vandermonde_zoh(np.array([g["a"]]), np.array([g["b"]]), np.array([g["c"]]),
                                 g["dt"], 2)
    assert abs(K[0] - g["k0"]) < 1e-10 and abs(K[1] - g["k1"]) < 1e-10


@pytest.mark.parametrize("N,L", [(1, 8), (4, 32), (16, 64)])
def test_zoh_vandermonde_equals_matrix_powers(N, L):
    rng = np.random.default_rng(80 + N)
    lam = -rng.uniform(0.05, 1, N) + 1j * rng.uniform(-20, 20, N)
    B, C = _cn(rng, N), _cn(rng, N)
    dt = 0.07
    d = [o.discretize_zoh_scalar(a, b, dt) for a, b in zip(lam, B)]
    Abar = np.diag([e[0] for e in d])
    Bbar = np.array([e[1] for e in d])
    ref = o.kernel_truncated(Abar, Bbar, C, L)
    K = o.kernel_vandermonde_zoh(lam, B, C, dt, L)
    np.testing.assert_allclose(K, ref, rtol=0, atol=1e-13 * np.abs(ref).max())
    # and it is the impulse response of the ZOH recurrence
    u = np.zeros(L)
    u[0] = 1.0
    np.testing.assert_allclose(o.recurrence(Abar, Bbar, C, 0.0, u), K, atol=1e-13 * np.abs(K).max())


def test_zoh_forward_and_recurrent_forward_agree():
    # with zero-order hold the kernel is not aliased, so the convolution and
    # the recurrence give the same outputs exactly (up to rounding)
    x = make_generic_inputs(H=2, N=6, L=40, batch=2, seed=82, diagonal=True)
    K, y = o.forward(x["lam"], None, None, x["B"], x["C"], x["dt"], x["D"], x["u"],
                     diagonal=True, disc="zoh")
    yr, _ = o.recurrent_forward(x["lam"], None, None, x["B"], x["C"], x["dt"], x["D"], x["u"],
                                diagonal=True, disc="zoh")
    np.testing.assert_allclose(y, yr, rtol=0, atol=1e-12 * np.abs(y).max())


def test_zoh_kernel_backward_finite_differences():
    x = make_generic_inputs(H=2, N=3, L=12, batch=1, seed=83, diagonal=True)
    x = {k: (None if v is None or k == "workload" else np.asarray(v, np.float64))
         for k, v in x.items()}
    dK = np.random.default_rng(84).standard_normal((2, 12))
    g = o.kernel_backward_dense(x["lam"], None, None, x["B"], x["C"], x["dt"], dK, diagonal=True,
                                disc="zoh")

    def loss(xx):
        K, _ = o.forward(xx["lam"], None, None, xx["B"], xx["C"], xx["dt"], np.zeros(2),
                         np.zeros((1, 2, 12)), diagonal=True, disc="zoh")
        return float(np.sum(K * dK))
    for name in ["lam", "B", "C", "dt"]:
        flat = x[name].reshape(-1)
        for i in range(flat.size):
            e = 1e-6 * max(1.0, abs(flat[i]))
            xp = {k: (None if v is None else v.copy()) for k, v in x.items()}
            xm = {k: (None if v is None else v.copy()) for k, v in x.items()}
            xp[name].reshape(-1)[i] += e
            xm[name].reshape(-1)[i] -= e
            fd = (loss(xp) - loss(xm)) / (2 * e)
            an = g[name].reshape(-1)[i]
            assert abs(fd - an) <= 1e-5 * max(1.0, abs(an)), (name, i, fd, an)


# --- The block: pre-norm, GLU-gated projection, residual ------------------------

def test_layer_norm_properties():
    rng = np.random.default_rng(90)
    x = 3.0 + 2.0 * rng.standard_normal((2, 7, 5))
    z = o.layer_norm(x, np.ones(7), np.zeros(7), eps=0.0)
    np.testing.assert_allclose(z.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose((z ** 2).mean(axis=1), 1.0, atol=1e-12)
    g, b = rng.standard_normal(7), rng.standard_normal(7)
    np.testing.assert_allclose(o.layer_norm(x, g, b, eps=0.0), z * g[None, :, None] + b[None, :, None],
                               atol=1e-12)
    # a constant column normalizes to the shift alone
    xc = np.ones((1, 7, 1)) * 4.2
    np.testing.assert_allclose(o.layer_norm(xc, g, b)[0, :, 0], b, atol=1e-12)


def test_glu_projection_closed_forms():
    rng = np.random.default_rng(91)
    H = 5
    s = rng.standard_normal((2, H, 4))
    # W = [I; 0], no bias: a = s, g = 0 -> s / 2
    W = np.vstack([np.eye(H), np.zeros((H, H))])
    np.testing.assert_allclose(o.glu_projection(s, W, np.zeros(2 * H)), s / 2, atol=1e-15)
    # a permutation in the value half moves channels: output channel c is s[perm[c]] / 2
    perm = np.array([3, 0, 4, 1, 2])
    Wp = np.vstack([np.eye(H)[perm], np.zeros((H, H))])
    np.testing.assert_allclose(o.glu_projection(s, Wp, np.zeros(2 * H)), s[:, perm] / 2, atol=1e-15)
    # W = 0: the output is the bias gate a sigmoid(g), the same at every position
    bias = rng.standard_normal(2 * H)
    out = o.glu_projection(s, np.zeros((2 * H, H)), bias)
    ref = bias[:H] / (1 + np.exp(-bias[H:]))
    np.testing.assert_allclose(out, np.broadcast_to(ref[None, :, None], out.shape), atol=1e-15)
    # the gate half: W = [0; I], bias = [1; 0] -> sigmoid(s)
    Wg = np.vstack([np.zeros((H, H)), np.eye(H)])
    bg = np.concatenate([np.ones(H), np.zeros(H)])
    np.testing.assert_allclose(o.glu_projection(s, Wg, bg), 1 / (1 + np.exp(-s)), atol=1e-15)


def test_block_forward_composition():
    # with W = [I; 0] and no bias the block is x + layer(layer_norm(x)) / 2
    x = make_generic_inputs(H=3, N=4, L=16, batch=2, seed=92)
    p = {"gamma": np.array([1.0, 0.5, 2.0]), "beta": np.array([0.0, 0.1, -0.2])}
    W = np.vstack([np.eye(3), np.zeros((3, 3))])
    out = o.block_forward(x["u"], p["gamma"], p["beta"], x["lam"], x["P"], x["Q"], x["B"],
                          x["C"], x["dt"], x["D"], W, np.zeros(6))
    z = o.layer_norm(x["u"], p["gamma"], p["beta"])
    _, s = o.forward(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], x["D"], z)
    np.testing.assert_allclose(out, x["u"] + s / 2, atol=1e-12)


# ---- rank-r low-rank term ([wiki] "Structured Transition Matrix": A = Lambda
# - P Q^* with low-rank P, Q; the correction by the Woodbury identity) --------

def _rank_case(N, r, seed, distinct_q):
    rng = np.random.default_rng(seed)
    cn = lambda *s: rng.normal(0, np.sqrt(0.5), s) + 1j * rng.normal(0, np.sqrt(0.5), s)
    lam = -rng.uniform(0.05, 1.0, N) + 1j * rng.uniform(-20, 20, N)
    P = cn(N, r)
    Q = 0.4 * cn(N, r) if distinct_q else P
    return lam, P, Q, cn(N), cn(N), float(np.exp(rng.uniform(np.log(1e-2), np.log(0.3))))


@pytest.mark.parametrize("r,distinct_q", [(2, False), (3, True), (4, False), (4, True)])
def test_lowrank_cauchy_equals_dense_aliased(r, distinct_q):
    # the plain definition (matrix powers of the dense bilinear system)
    # against the Cauchy sums + r x r Woodbury solve, on the same A
    N, L = 12, 64
    lam, P, Q, B, C, dt = _rank_case(N, r, 100 + r, distinct_q)
    K = np.fft.ifft(o.generating_function_lowrank(lam, P, Q, B, C, dt, L)).real
    Abar, Bbar = o.discretize_bilinear(o.dense_state_matrix(lam, P, Q), B, dt)
    Kd = o.kernel_aliased_dense(Abar, Bbar, C, L)
    assert np.abs(K - Kd).max() <= 1e-10 * np.abs(Kd).max()


@pytest.mark.parametrize("r", [2, 3])
def test_lowrank_generating_function_equals_resolvent_solve(r):
    # K-hat_l = 2/(1+z) C (g I - A)^{-1} B by a dense linear solve at every
    # regular root of unity, and the closed-form limit at z = -1
    N, L = 9, 32
    lam, P, Q, B, C, dt = _rank_case(N, r, 200 + r, True)
    # A written out as the diagonal minus r rank-one terms
    A = np.diag(lam) - sum(np.outer(P[:, j], Q[:, j].conj()) for j in range(r))
    kh = o.generating_function_lowrank(lam, P, Q, B, C, dt, L)
    for l in range(L):
        if 2 * l == L:
            assert abs(kh[l] - dt / 2 * np.sum(C * B)) <= 1e-13 * np.abs(kh).max()
            continue
        z = np.exp(-2j * np.pi * l / L)
        g = 2 / dt * (1 - z) / (1 + z)
        ref = 2 / (1 + z) * (C @ np.linalg.solve(g * np.eye(N) - A, B))
        assert abs(kh[l] - ref) <= 1e-11 * abs(ref) + 1e-13


def test_lowrank_zero_column_reduces_the_rank():
    # a zero column of P (with any Q) or of Q removes that rank-one term
    N, L = 10, 48
    lam, P, Q, B, C, dt = _rank_case(N, 3, 300, True)
    for j in range(3):
        keep = [i for i in range(3) if i != j]
        Pz = P.copy()
        Pz[:, j] = 0
        ref = o.generating_function_lowrank(lam, P[:, keep], Q[:, keep], B, C, dt, L)
        got = o.generating_function_lowrank(lam, Pz, Q, B, C, dt, L)
        assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()
        Qz = Q.copy()
        Qz[:, j] = 0
        got = o.generating_function_lowrank(lam, P, Qz, B, C, dt, L)
        assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()
    # all columns zero: the diagonal system
    Z = np.zeros((N, 3), np.complex128)
    diag = o.generating_function(lam, np.zeros(N), np.zeros(N), B, C, dt, L)
    assert np.abs(o.generating_function_lowrank(lam, Z, Q, B, C, dt, L) - diag).max() \
        <= 1e-13 * np.abs(diag).max()


def test_lowrank_rank_one_and_column_order():
    # r = 1 is the rank-1 generating function; permuting the columns of P and
    # Q together leaves P Q^* (and so K-hat) unchanged
    N, L = 16, 64
    lam, P, Q, B, C, dt = _rank_case(N, 1, 400, True)
    ref = o.generating_function(lam, P[:, 0], Q[:, 0], B, C, dt, L)
    got = o.generating_function_lowrank(lam, P, Q, B, C, dt, L)
    assert np.abs(got - ref).max() <= 1e-13 * np.abs(ref).max()
    lam, P, Q, B, C, dt = _rank_case(N, 4, 401, True)
    perm = [2, 0, 3, 1]
    a = o.generating_function_lowrank(lam, P, Q, B, C, dt, L)
    b = o.generating_function_lowrank(lam, P[:, perm], Q[:, perm], B, C, dt, L)
    assert np.abs(a - b).max() <= 1e-12 * np.abs(a).max()


@pytest.mark.parametrize("L", [16, 256])
def test_lowrank_dc_and_nyquist_sums(L):
    # sum_k K_k = Re K-hat(1) = Re(-C A^{-1} B); sum_k (-1)^k K_k = Re((dt/2) C.B)
    N = 8
    lam, P, Q, B, C, dt = _rank_case(N, 2, 500 + L, True)
    K = np.fft.ifft(o.generating_function_lowrank(lam, P, Q, B, C, dt, L)).real
    A = o.dense_state_matrix(lam, P, Q)
    dc = (-C @ np.linalg.solve(A, B)).real
    assert abs(K.sum() - dc) <= 1e-11 * max(1.0, abs(dc))
    ny = (dt / 2 * np.sum(C * B)).real
    assert abs(np.sum(K * (-1.0) ** np.arange(L)) - ny) <= 1e-11 * max(1.0, abs(ny))


def test_lowrank_forward_layout():
    # the (H, r, N, 2) storage: forward() per channel equals the per-channel
    # generating function of the N x r matrices
    x = make_generic_inputs(H=2, N=8, L=32, batch=2, seed=600, rank=3, distinct_q=True)
    K, y = o.forward(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], x["D"], x["u"])
    c = lambda a: a[..., 0].astype(np.float64) + 1j * a[..., 1]
    for h in range(2):
        Pm, Qm = c(x["P"][h]).T, c(x["Q"][h]).T         # (N, r)
        Abar, Bbar = o.discretize_bilinear(o.dense_state_matrix(c(x["lam"][h]), Pm, Qm),
                                           c(x["B"][h]), float(x["dt"][h]))
        Kd = o.kernel_aliased_dense(Abar, Bbar, c(x["C"][h]), 32)
        assert np.abs(K[h] - Kd).max() <= 1e-10 * np.abs(Kd).max()
