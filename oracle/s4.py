"""fp64 reference implementation of the S4 DPLR convolution-mode forward pass.

TEST INFRASTRUCTURE ONLY: this module is the oracle that the GPU library is
checked against.  It is imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark, and by nothing else.  It shares no code,
tables or constants with the HIP path; both sides only share the seeded input
generator in ``synth/``.

Everything here is written for a reader to check against the pages by eye:
plain NumPy in float64/complex128, no blocking or fusion, library routines
(matrix products, solves, eigh, FFT) only as whole steps.

Pages cited (by title and section):
  [scratch]   "The S4 kernel, from scratch" -- section 1 (continuous SSM),
              2 (HiPPO initialization -> DPLR form), 3 (Discretization),
              4 (The convolutional kernel via the generating function, with
              its "Aliasing" paragraph), 5 (Two views, kept in sync),
              6 (Trainable layer).
  [wiki]      "S4" wiki page -- "Structured Transition Matrix", "S4D".
  [glossary]  "Structured state-space sequence model and S4" -- "One linear
              layer, two computational views", "Follow one input through
              memory" (worked-example table).
  [kronos]    "Structured State-Space Models (S4)" -- "A linear system as a
              layer", "Recurrence and convolution duality".

Readings of points the pages leave open (numbered as in the design notes):
  R1  the HiPPO-LegS entries are not printed; the standard LegS matrix is used.
  R2  the rank-1 NPLR factor is P_n = sqrt(n + 1/2).
  R3  eigh is taken of -i*T (T the skew part); eigenvalues ascending; each
      eigenvector rephased so that (V^* P)_n is real and >= 0.
  R5  the kernel is the real part of the inverse FFT (C is complex).
  R6  C-bar = C: the length-L inverse FFT yields the *aliased* kernel.
  R7  bilinear B-bar = (I - dt/2 A)^{-1} dt B.
  R8  z_l = exp(-2 pi i l / L); inverse FFT scaled by 1/L (NumPy convention).
  R9  at z = -1 (l = L/2) the generating function takes its limit
      (dt/2) * sum_n C_n B_n.
  R10 y_t = sum_{j<=t} K_j u_{t-j} + D u_t (no one-step delay).
  R12 the causal convolution is zero-padded to exactly 2L.
  R13 ZOH uses the expm1 form (limit dt*b at a = 0); the pages' Taylor
      threshold is not reproduced (parity unpinned for that threshold, which
      no hot-path result depends on).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "hippo_legs", "nplr_legs", "dplr_legs",
    "dense_state_matrix", "discretize_bilinear", "discretize_zoh_scalar",
    "kernel_truncated", "kernel_aliased_dense", "generating_function",
    "generating_function_lowrank",
    "kernel_cauchy", "conv_direct", "conv_direct_at", "conv_fft",
    "recurrence", "forward", "recurrent_forward",
    "conv_backward_direct", "conv_backward_fft", "kernel_backward_dense",
    "kernel_vandermonde_zoh", "layer_norm", "glu_projection", "block_forward",
]


# ---------------------------------------------------------------------------
# Initialization: HiPPO-LegS -> NPLR -> DPLR   ([scratch] section 2;
# [wiki] "Structured Transition Matrix")
# ---------------------------------------------------------------------------

def hippo_legs(N: int):
    """HiPPO-LegS state matrix A (N x N, real) and input vector B (N).

    [scratch] section 2 names the matrix but does not print it (reading R1):
    A[n,k] = -sqrt((2n+1)(2k+1)) below the diagonal, -(n+1) on it, 0 above;
    B[n] = sqrt(2n+1).
    """
    n = np.arange(N, dtype=np.float64)
    A = np.zeros((N, N), dtype=np.float64)
    for i in range(N):
        for k in range(N):
            if i > k:
                A[i, k] = -np.sqrt((2 * n[i] + 1) * (2 * n[k] + 1))
            elif i == k:
                A[i, k] = -(n[i] + 1)
    B = np.sqrt(2 * n + 1)
    return A, B


def nplr_legs(N: int):
    """Normal-plus-low-rank split A = A_normal - P P^T ([scratch] section 2).

    Returns (A, P, B, S) with S = A + P P^T the normal part (reading R2:
    P_n = sqrt(n + 1/2), which makes S = -I/2 + skew-symmetric).
    """
    A, B = hippo_legs(N)
    P = np.sqrt(np.arange(N, dtype=np.float64) + 0.5)
    S = A + np.outer(P, P)
    return A, P, B, S


def dplr_legs(N: int):
    """DPLR parameters (Lambda, P~, B~, V) with A = V (Lambda - P~ P~^*) V^*.

    [scratch] section 2: diagonalize the normal part with a Hermitian eigh and
    rotate P and B into the eigenbasis; Q = P.  Reading R3 fixes the basis:
    eigh of -i*T, ascending eigenvalues, eigenvectors rephased so that every
    P~_n is real and non-negative.
    """
    A, P, B, S = nplr_legs(N)
    T = S + 0.5 * np.eye(N)                 # skew-symmetric part of S
    mu, V = np.linalg.eigh(-1j * T)         # -iT is Hermitian; mu ascending
    Pt = V.conj().T @ P
    phase = np.exp(1j * np.angle(Pt))
    phase[np.abs(Pt) == 0] = 1.0
    V = V * phase[None, :]                  # column n times e^{i arg P~_n}
    lam = -0.5 + 1j * mu                    # eigenvalues of S = -I/2 + T
    Pt = V.conj().T @ P
    Bt = V.conj().T @ B
    return lam, Pt, Bt, V


# ---------------------------------------------------------------------------
# Dense system and discretization   ([scratch] sections 1 and 3)
# ---------------------------------------------------------------------------

def dense_state_matrix(lam, P, Q):
    """A = diag(Lambda) - P Q^*  ([scratch] section 2; [wiki] "Structured
    Transition Matrix": A = Lambda - P Q^* with low-rank P, Q).

    P, Q are vectors (rank 1) or N x r matrices (rank r)."""
    lam = np.asarray(lam, dtype=np.complex128)
    P = np.asarray(P, np.complex128)
    Q = np.asarray(Q, np.complex128)
    if P.ndim == 1:
        return np.diag(lam) - np.outer(P, np.conj(Q))
    return np.diag(lam) - P @ np.conj(Q).T


def discretize_bilinear(A, B, dt):
    """Bilinear (Tustin) discretization ([scratch] section 3; reading R7).

    A-bar = (I - dt/2 A)^{-1} (I + dt/2 A),  B-bar = (I - dt/2 A)^{-1} dt B.
    """
    A = np.asarray(A, dtype=np.complex128)
    I = np.eye(A.shape[0], dtype=np.complex128)
    M = I - (dt / 2.0) * A
    Abar = np.linalg.solve(M, I + (dt / 2.0) * A)
    Bbar = np.linalg.solve(M, dt * np.asarray(B, dtype=np.complex128))
    return Abar, Bbar


def discretize_zoh_scalar(a, b, dt):
    """Zero-order hold for a scalar system: A-bar = exp(dt a),
    B-bar = (exp(dt a) - 1)/a * b  ([scratch] section 3; [glossary] "Follow one
    input through memory").  Reading R13: expm1 form, limit dt*b at a = 0."""
    if a == 0:
        return 1.0, dt * b
    return np.exp(dt * a), np.expm1(dt * a) / a * b


# ---------------------------------------------------------------------------
# Convolution kernel: plain definition   ([scratch] section 4)
# ---------------------------------------------------------------------------

def kernel_truncated(Abar, Bbar, C, L):
    """K_k = Re(C A-bar^k B-bar), k < L: the first L Markov parameters
    ([scratch] section 4 kernel definition; [glossary] k_j = C A-bar^j B-bar).
    Computed by repeated multiplication, one power at a time."""
    C = np.asarray(C, dtype=np.complex128)
    x = np.asarray(Bbar, dtype=np.complex128).copy()
    K = np.empty(L, dtype=np.float64)
    for k in range(L):
        K[k] = (C @ x).real
        x = Abar @ x
    return K


def kernel_aliased_dense(Abar, Bbar, C, L):
    """The aliased kernel sum_j K_{k+jL} = Re(C A-bar^k (I - A-bar^L)^{-1} B-bar).

    [scratch] section 4, "Aliasing": the length-L inverse FFT of the generating
    function returns the kernel summed over all periods.  The geometric series
    over periods is summed in closed form with one linear solve (readings R5,
    R6), then the powers are taken one at a time as in ``kernel_truncated``.
    """
    Abar = np.asarray(Abar, dtype=np.complex128)
    N = Abar.shape[0]
    AL = np.linalg.matrix_power(Abar, L)
    x0 = np.linalg.solve(np.eye(N) - AL, np.asarray(Bbar, dtype=np.complex128))
    return kernel_truncated(Abar, x0, C, L)


def kernel_vandermonde_zoh(lam, B, C, dt, L):
    """Kernel of a diagonal system ([wiki] "S4D": A = diag(a_n)) discretized by
    zero-order hold ([scratch] section 3: A-bar_n = exp(dt a_n); B-bar_n from
    ``discretize_zoh_scalar``), as the Vandermonde product of its definition
    K_k = Re(sum_n C_n B-bar_n A-bar_n^k), k = 0 .. L-1 ([scratch] section 4,
    the powers written out).  This is the kernel itself, not an aliased one."""
    lam = np.asarray(lam, np.complex128)
    disc = [discretize_zoh_scalar(a, b, dt) for a, b in zip(lam, np.asarray(B, np.complex128))]
    Abar = np.array([d[0] for d in disc], dtype=np.complex128)
    Bbar = np.array([d[1] for d in disc], dtype=np.complex128)
    k = np.arange(L)
    V = Abar[None, :] ** k[:, None]                     # Vandermonde matrix [L][N]
    return (V @ (np.asarray(C, np.complex128) * Bbar)).real


# ---------------------------------------------------------------------------
# Convolution kernel: the pages' method   ([scratch] section 4)
# ---------------------------------------------------------------------------

def generating_function(lam, P, Q, B, C, dt, L):
    """K-hat at the L roots of unity by four Cauchy sums and a rank-1
    Woodbury correction ([scratch] section 4 equations; [wiki] "Structured
    Transition Matrix").

    z_l = exp(-2 pi i l/L) (reading R8); g = (2/dt)(1-z)/(1+z);
    k_ab = sum_n w_n / (g - Lambda_n) with weights C*B, C*P, conj(Q)*B,
    conj(Q)*P; K-hat = 2/(1+z) * (k00 - k01 k10 / (1 + k11)).
    At l = L/2 (z = -1) the limit (dt/2) sum_n C_n B_n is used (reading R9).
    """
    lam = np.asarray(lam, np.complex128)
    P = np.asarray(P, np.complex128)
    Q = np.asarray(Q, np.complex128)
    B = np.asarray(B, np.complex128)
    C = np.asarray(C, np.complex128)
    ell = np.arange(L)
    Khat = np.empty(L, dtype=np.complex128)
    regular = np.ones(L, dtype=bool)
    if L % 2 == 0:
        regular[L // 2] = False
    z = np.exp(-2j * np.pi * ell[regular] / L)
    g = (2.0 / dt) * (1.0 - z) / (1.0 + z)
    r = 1.0 / (g[:, None] - lam[None, :])          # Cauchy matrix [l, n]
    k00 = r @ (C * B)
    k01 = r @ (C * P)
    k10 = r @ (np.conj(Q) * B)
    k11 = r @ (np.conj(Q) * P)
    Khat[regular] = (2.0 / (1.0 + z)) * (k00 - k01 * k10 / (1.0 + k11))
    if L % 2 == 0:
        Khat[L // 2] = (dt / 2.0) * np.sum(C * B)
    return Khat


def generating_function_lowrank(lam, P, Q, B, C, dt, L):
    """K-hat at the L roots of unity for a rank-r low-rank term, A = Lambda -
    P Q^* with P, Q of shape (N, r) ([wiki] "Structured Transition Matrix":
    low-rank P, Q, the correction handled by the Woodbury identity;
    [scratch] section 4 for g, the roots of unity and the 2/(1+z) factor).

    With R = (g I - Lambda)^{-1} diagonal, the Woodbury identity gives
      C (g I - A)^{-1} B = k00 - k01 (I_r + k11)^{-1} k10,
    k00 = C R B (scalar), k01 = C R P (1 x r), k10 = Q^* R B (r x 1),
    k11 = Q^* R P (r x r): (r + 1)^2 Cauchy sums over the poles.  The r x r
    system is solved per frequency by a library solve.  At z = -1 the limit
    (dt/2) sum_n C_n B_n (reading R9: the correction vanishes like 1/g^2).
    For r = 1 this is ``generating_function``."""
    lam = np.asarray(lam, np.complex128)
    P = np.asarray(P, np.complex128)
    Q = np.asarray(Q, np.complex128)
    B = np.asarray(B, np.complex128)
    C = np.asarray(C, np.complex128)
    r_rank = P.shape[1]
    ell = np.arange(L)
    Khat = np.empty(L, dtype=np.complex128)
    regular = np.ones(L, dtype=bool)
    if L % 2 == 0:
        regular[L // 2] = False
    z = np.exp(-2j * np.pi * ell[regular] / L)
    g = (2.0 / dt) * (1.0 - z) / (1.0 + z)
    R = 1.0 / (g[:, None] - lam[None, :])               # Cauchy matrix [l, n]
    k00 = R @ (C * B)                                   # [l]
    k01 = R @ (C[:, None] * P)                          # [l, r]
    k10 = R @ (np.conj(Q) * B[:, None])                 # [l, r]
    k11 = np.einsum("ln,ni,nj->lij", R, np.conj(Q), P)  # [l, r, r]
    I = np.eye(r_rank, dtype=np.complex128)
    x = np.linalg.solve(I[None] + k11, k10[..., None])[..., 0]   # (I + k11)^{-1} k10
    Khat[regular] = (2.0 / (1.0 + z)) * (k00 - np.sum(k01 * x, axis=1))
    if L % 2 == 0:
        Khat[L // 2] = (dt / 2.0) * np.sum(C * B)
    return Khat


def kernel_cauchy(lam, P, Q, B, C, dt, L):
    """Time-domain kernel K = Re(ifft(K-hat)) ([scratch] section 4: the
    length-L inverse FFT of the generating function gives the kernel in time;
    readings R5, R8)."""
    if np.ndim(P) == 2:
        return np.fft.ifft(generating_function_lowrank(lam, P, Q, B, C, dt, L)).real
    return np.fft.ifft(generating_function(lam, P, Q, B, C, dt, L)).real


# ---------------------------------------------------------------------------
# The two views   ([scratch] section 5; [glossary] "One linear layer, two
# computational views"; [kronos] "Recurrence and convolution duality")
# ---------------------------------------------------------------------------

def conv_direct(u, K, D):
    """y_t = sum_{j=0}^{t} K_j u_{t-j} + D u_t, summed directly (O(L^2)).

    [scratch] section 1 (feed-through D) and section 4 (y = K * u); reading R10.
    """
    u = np.asarray(u, np.float64)
    K = np.asarray(K, np.float64)
    L = u.shape[0]
    y = np.empty(L, dtype=np.float64)
    for t in range(L):
        y[t] = np.dot(K[: t + 1], u[t::-1]) + D * u[t]
    return y


def conv_direct_at(u, K, D, t):
    """One output sample y_t of ``conv_direct``."""
    u = np.asarray(u, np.float64)
    K = np.asarray(K, np.float64)
    return float(np.dot(K[: t + 1], u[t::-1]) + D * u[t])


def conv_fft(u, K, D):
    """Causal convolution by an FFT zero-padded to 2L ([scratch] section 5:
    the padding keeps the circular product from wrapping the tail of the
    output onto its start; reading R12), plus D u.

    ``u`` may be [..., L]; ``K`` broadcasts against it; ``D`` likewise
    (shape [..., 1] or scalar).
    """
    u = np.asarray(u, np.float64)
    K = np.asarray(K, np.float64)
    L = u.shape[-1]
    n = 2 * L
    y = np.fft.irfft(np.fft.rfft(u, n) * np.fft.rfft(K, n), n)[..., :L]
    return y + np.asarray(D, np.float64) * u


def recurrence(Abar, Bbar, C, D, u, x0=None, return_state=False):
    """Recurrent view x_t = A-bar x_{t-1} + B-bar u_t, y_t = Re(C x_t) + D u_t
    ([scratch] section 5; [glossary] h_t = A-bar h_{t-1} + B-bar u_t).

    u is (..., T): every leading index is an independent sequence of the same
    system.  The state before the first step is x0 (..., N), zero if None.
    With return_state the state after the last step is returned as well.
    """
    Abar = np.asarray(Abar, np.complex128)
    Bbar = np.asarray(Bbar, np.complex128)
    C = np.asarray(C, np.complex128)
    u = np.asarray(u, np.float64)
    N = Abar.shape[0]
    x = np.zeros(u.shape[:-1] + (N,), dtype=np.complex128)
    if x0 is not None:
        x = x + np.asarray(x0, np.complex128)
    y = np.empty(u.shape, dtype=np.float64)
    for t in range(u.shape[-1]):
        ut = u[..., t]
        x = x @ Abar.T + Bbar * ut[..., None]
        y[..., t] = (x @ C).real + D * ut
    return (y, x) if return_state else y


# ---------------------------------------------------------------------------
# Whole forward pass over channels and batch
# ---------------------------------------------------------------------------

def _as_complex(a):
    """(..., 2) float -> complex128 (the interleaved layout of [scratch]
    section 6: complex parameters stored as real (..., 2) tensors)."""
    a = np.asarray(a, dtype=np.float64)
    return a[..., 0] + 1j * a[..., 1]


def _low_rank(a):
    """P or Q as stored, (H, N, 2) for rank 1 or (H, r, N, 2) for rank r
    (the r vectors of length N one after another), -> complex (H, N) or
    (H, N, r): per channel the N x r matrix of [wiki] "Structured Transition
    Matrix"."""
    c = _as_complex(a)
    return c if c.ndim == 2 else np.swapaxes(c, 1, 2)


def forward(lam, P, Q, B, C, dt, D, u, method="cauchy", diagonal=False, disc="bilinear"):
    """K [H, L] and y [batch, H, L] for H independent channels
    ([scratch] section 1: one SSM per feature channel).

    Complex inputs are (H, N, 2) float arrays (P and Q may be (H, r, N, 2)
    for a rank-r low-rank term); dt, D are (H,); u is (batch, H, L).  ``method`` selects the kernel: "cauchy" (the pages'
    generating-function method) or "dense" (the aliased plain definition).
    ``diagonal`` drops the low-rank term (S4D, [wiki] "S4D": P = Q = 0).
    ``disc="zoh"`` (diagonal only) uses the zero-order-hold Vandermonde kernel
    of ``kernel_vandermonde_zoh`` instead.
    """
    if disc == "zoh":
        if not diagonal:
            raise ValueError("zero-order hold is defined here for diagonal systems only")
        lam_c, B_c, C_c = _as_complex(lam), _as_complex(B), _as_complex(C)
        dts = np.asarray(dt, np.float64)
        u = np.asarray(u, np.float64)
        L = u.shape[-1]
        K = np.stack([kernel_vandermonde_zoh(lam_c[h], B_c[h], C_c[h], dts[h], L)
                      for h in range(lam_c.shape[0])])
        Dv = np.zeros(lam_c.shape[0]) if D is None else np.asarray(D, np.float64)
        return K, conv_fft(u, K[None, :, :], Dv[None, :, None])
    lam_c = _as_complex(lam)
    H, N = lam_c.shape
    u = np.asarray(u, np.float64)
    L = u.shape[-1]
    if diagonal:
        P_c = np.zeros((H, N), np.complex128)
        Q_c = P_c
    else:
        P_c = _low_rank(P)
        Q_c = P_c if Q is None else _low_rank(Q)
    B_c = _as_complex(B)
    C_c = _as_complex(C)
    dt = np.asarray(dt, np.float64)
    D = np.zeros(H) if D is None else np.asarray(D, np.float64)
    K = np.empty((H, L), dtype=np.float64)
    for h in range(H):
        if method == "cauchy":
            K[h] = kernel_cauchy(lam_c[h], P_c[h], Q_c[h], B_c[h], C_c[h], dt[h], L)
        elif method == "dense":
            A = dense_state_matrix(lam_c[h], P_c[h], Q_c[h])
            Abar, Bbar = discretize_bilinear(A, B_c[h], dt[h])
            K[h] = kernel_aliased_dense(Abar, Bbar, C_c[h], L)
        else:
            raise ValueError(method)
    y = conv_fft(u, K[None, :, :], D[None, :, None])
    return K, y


def recurrent_forward(lam, P, Q, B, C, dt, D, u, x0=None, diagonal=False, disc="bilinear"):
    """The recurrent view over channels and batch: y [batch, H, T] and the
    final state [batch, H, N] (complex), from the dense bilinear A-bar, B-bar
    of A = Lambda - P Q^* ([scratch] sections 3 and 5; [wiki] "Structured
    Transition Matrix").  Inputs as for ``forward``; x0 is [batch, H, N]
    complex or None (zero).  ``diagonal`` drops the low-rank term."""
    lam_c = _as_complex(lam)
    H, N = lam_c.shape
    u = np.asarray(u, np.float64)
    if diagonal:
        P_c = np.zeros((H, N), np.complex128)
        Q_c = P_c
    else:
        P_c = _low_rank(P)
        Q_c = P_c if Q is None else _low_rank(Q)
    B_c = _as_complex(B)
    C_c = _as_complex(C)
    dt = np.asarray(dt, np.float64)
    D = np.zeros(H) if D is None else np.asarray(D, np.float64)
    y = np.empty(u.shape, dtype=np.float64)
    xT = np.empty((u.shape[0], H, N), dtype=np.complex128)
    for h in range(H):
        if disc == "zoh":
            if not diagonal:
                raise ValueError("zero-order hold is defined here for diagonal systems only")
            d = [discretize_zoh_scalar(a, b, dt[h]) for a, b in zip(lam_c[h], B_c[h])]
            Abar = np.diag([e[0] for e in d]).astype(np.complex128)
            Bbar = np.array([e[1] for e in d], dtype=np.complex128)
        else:
            A = dense_state_matrix(lam_c[h], P_c[h], Q_c[h])
            Abar, Bbar = discretize_bilinear(A, B_c[h], dt[h])
        y[:, h], xT[:, h] = recurrence(Abar, Bbar, C_c[h], D[h], u[:, h],
                                       None if x0 is None else x0[:, h], return_state=True)
    return y, xT


# ---------------------------------------------------------------------------
# Backward pass of the convolution-mode forward   ([scratch] sections 5 and 6:
# the layer is trained through the convolution; its parameters are
# Lambda, P, B, C, dt, D)
# ---------------------------------------------------------------------------

def conv_backward_direct(u, K, D, dy):
    """Gradients of a scalar loss through y = K * u + D u, given dy = dloss/dy,
    by direct summation of their plain definitions:

      du[b,h,t] = sum_{j=0}^{L-1-t} K[h,j] dy[b,h,t+j] + D[h] dy[b,h,t]
      dK[h,j]   = sum_b sum_{t=j}^{L-1} dy[b,h,t] u[b,h,t-j]
      dD[h]     = sum_b sum_t dy[b,h,t] u[b,h,t]

    u, dy: (batch, H, L); K: (H, L); D: (H,).  Returns (du, dK, dD).
    O(B H L^2): for small inputs."""
    u = np.asarray(u, np.float64)
    dy = np.asarray(dy, np.float64)
    K = np.asarray(K, np.float64)
    D = np.asarray(D, np.float64)
    L = u.shape[-1]
    du = D[None, :, None] * dy
    dK = np.zeros(K.shape, np.float64)
    for j in range(L):
        du[..., : L - j] += K[None, :, j, None] * dy[..., j:]
        dK[:, j] = np.sum(dy[..., j:] * u[..., : L - j], axis=(0, 2))
    dD = np.sum(dy * u, axis=(0, 2))
    return du, dK, dD


def conv_backward_fft(u, K, D, dy):
    """The same three gradients through fp64 FFTs of length 2L (library
    routine): du is the correlation of dy with K, dK the correlation of dy
    with u summed over the batch (zero padding to 2L leaves no wrap-around)."""
    u = np.asarray(u, np.float64)
    dy = np.asarray(dy, np.float64)
    K = np.asarray(K, np.float64)
    D = np.asarray(D, np.float64)
    L = u.shape[-1]
    n = 2 * L
    Fy = np.fft.rfft(dy, n)
    du = np.fft.irfft(Fy * np.conj(np.fft.rfft(K, n))[None], n)[..., :L] + D[None, :, None] * dy
    dK = np.fft.irfft(np.sum(Fy * np.conj(np.fft.rfft(u, n)), axis=0), n)[..., :L]
    dD = np.sum(dy * u, axis=(0, 2))
    return du, dK, dD


def kernel_backward_dense(lam, P, Q, B, C, dt, dK, diagonal=False, disc="bilinear"):
    """Gradients of loss = sum_{h,k} dK[h,k] K[h,k] with respect to the
    kernel's parameters, where K is the plain aliased definition
    K_k = Re(C A-bar^k (I - A-bar^L)^{-1} B-bar) of the dense bilinear system
    for A = Lambda - P Q^* ([scratch] sections 3 and 4; [wiki] "Structured
    Transition Matrix").  The derivative is taken by PyTorch's reverse-mode
    differentiation (fp64, CPU) of that definition, with every complex
    parameter held as its real and imaginary parts.

    Inputs as for ``forward``; dK is (H, L).  Returns a dict of gradients in
    the same (..., 2) layout: "lam", "B", "C", "dt" and, unless diagonal,
    "P" and "Q" -- with Q None (Q = P) the P gradient includes the Q path
    and "Q" is None."""
    import torch
    dK = np.asarray(dK, np.float64)
    H, L = dK.shape
    tied = Q is None
    t = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    lam_t, B_t, C_t = t(lam), t(B), t(C)
    dt_t = t(dt)
    P_t = None if diagonal else t(P)
    Q_t = None if (diagonal or tied) else t(Q)
    cx = lambda a: torch.complex(a[..., 0], a[..., 1])
    N = lam_t.shape[1]
    eye = torch.eye(N, dtype=torch.complex128)
    loss = torch.zeros((), dtype=torch.float64)
    for h in range(H):
        lam_c, B_c, C_c = cx(lam_t[h]), cx(B_t[h]), cx(C_t[h])
        if disc == "zoh":
            # the Vandermonde definition of kernel_vandermonde_zoh (diagonal only)
            z = dt_t[h] * lam_c
            Bbar = torch.expm1(z) / lam_c * B_c
            k = torch.arange(L, dtype=torch.float64)
            V = torch.exp(k[:, None] * z[None, :])
            Kh = (V @ (C_c * Bbar)).real
            loss = loss + torch.sum(Kh * torch.from_numpy(dK[h]))
            continue
        A = torch.diag(lam_c)
        if not diagonal:
            P_c = cx(P_t[h])
            Q_c = P_c if tied else cx(Q_t[h])
            A = A - torch.outer(P_c, Q_c.conj())
        half = dt_t[h] / 2
        M = eye - half * A
        Abar = torch.linalg.solve(M, eye + half * A)
        Bbar = torch.linalg.solve(M, (dt_t[h] * B_c)[:, None])[:, 0]
        ApowL = torch.linalg.matrix_power(Abar, L)
        x = torch.linalg.solve(eye - ApowL, Bbar[:, None])[:, 0]
        Ks = []
        for k in range(L):
            Ks.append((C_c @ x).real)
            x = Abar @ x
        loss = loss + torch.sum(torch.stack(Ks) * torch.from_numpy(dK[h]))
    loss.backward()
    g = lambda a: None if a is None else a.grad.numpy().copy()
    return {"lam": g(lam_t), "P": g(P_t), "Q": g(Q_t), "B": g(B_t), "C": g(C_t),
            "dt": g(dt_t)}


# ---------------------------------------------------------------------------
# The block around the layer   ([scratch] section 6: the block adds a
# pre-norm, a GLU-gated projection and a residual connection)
# ---------------------------------------------------------------------------

def layer_norm(x, gamma, beta, eps=1e-5):
    """Normalization over the H channels at every (batch, time) position
    (reading: layer normalization with the biased variance, eps = 1e-5, and a
    per-channel gain and shift).  x: (batch, H, L)."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    g = np.asarray(gamma, np.float64)[None, :, None]
    b = np.asarray(beta, np.float64)[None, :, None]
    return (x - mu) / np.sqrt(var + eps) * g + b


def glu_projection(s, W, bias):
    """[a; g] = W s + bias over the channels (W: (2H, H)), then the gated
    linear unit a * sigmoid(g) (reading: the first H outputs are the values,
    the last H the gates).  s: (batch, H, L) -> (batch, H, L)."""
    s = np.asarray(s, np.float64)
    W = np.asarray(W, np.float64)
    H = s.shape[1]
    z = np.matmul(W[None], s) + np.asarray(bias, np.float64)[None, :, None]
    a, g = z[:, :H], z[:, H:]
    return a / (1.0 + np.exp(-g))


def block_forward(x, gamma, beta, lam, P, Q, B, C, dt, D, W, bias, diagonal=False,
                  disc="bilinear"):
    """out = x + GLU(W s + bias), s = the layer applied to layer_norm(x)
    ([scratch] section 6; readings: no activation between the layer and the
    projection, no dropout)."""
    z = layer_norm(x, gamma, beta)
    _, s = forward(lam, P, Q, B, C, dt, D, z, diagonal=diagonal, disc=disc)
    return np.asarray(x, np.float64) + glu_projection(s, W, bias)
