"""Host checks of the half-length inverse used for L = 32768 and 65536 at rank 1.

The time-domain kernel K = Re IDFT_L(X) / L of a generating function X
("The S4 kernel, from scratch", section 4: the kernel is read off the
generating function at the L roots of unity by an inverse FFT) is recovered
from the L/2-point spectrum
    Y_m = (Xh_m + Xh_{m+L/2}) + i e^{2 pi i m/L} (Xh_m - Xh_{m+L/2}),
    Xh_m = (X_m + conj X_{L-m}) / 2,
as K_2n + i K_2n+1 = IDFT_{L/2}(Y)_n / L.  The GPU kernel forms Y from lane
pairs; these tests check the identity against numpy's FFT and that the
kernel's thread-to-frequency map (restated here) writes every Y slot once.

The padded spectrum S_k = sum_{n<L} K_n e^{-i pi k n / L} + D (k <= L) then
comes without an L-point transform: the even bins are the Hermitian part,
S_2m = Xh_m + D, and the odd bins come from F = DFT_{L/2}(z_m e^{-2 pi i m/L})
through E_j = (F_j + conj F_p) / 2, O_j = (F_j - conj F_p) / (2i),
p = L/2 - 1 - j, S_{2j+1} = E_j + e^{-i pi (2j+1)/L} O_j + D
("The S4 kernel, from scratch", section 5: the kernel's spectrum zero-padded
to 2L).  test_padded_spectrum_from_y checks that chain against numpy's rfft.
"""
import numpy as np
import pytest


def _y_from_x(X):
    L = X.shape[0]
    m = np.arange(L // 2)
    xh = 0.5 * (X + np.conj(X[(-np.arange(L)) % L]))
    a, b = xh[m], xh[m + L // 2]
    return (a + b) + 1j * np.exp(2j * np.pi * m / L) * (a - b)


@pytest.mark.parametrize("L", [8, 64, 32768, 65536])
def test_identity(L):
    rng = np.random.default_rng(L)
    X = rng.standard_normal(L) + 1j * rng.standard_normal(L)
    K = np.fft.ifft(X).real                      # Re IDFT_L(X) / L
    z = np.fft.ifft(_y_from_x(X)) * (L // 2) / L  # unnormalized IDFT_{L/2}(Y) / L
    np.testing.assert_allclose(z.real, K[0::2], atol=1e-15 * np.abs(K).max() * 10)
    np.testing.assert_allclose(z.imag, K[1::2], atol=1e-15 * np.abs(K).max() * 10)


@pytest.mark.parametrize("L", [32768, 65536])
def test_lane_pair_map(L):
    M1, H2, Q = L // 512, L // 2, L // 4
    g = np.arange(L // 2)
    odd = g & 1
    q = g >> 1
    l = (q >> 7) + M1 * (q & 127)
    assert l.min() == 0 and l.max() < Q
    f0 = np.where(l == 0, np.where(odd, Q, 0), np.where(odd, H2 - l, l))
    f1 = np.where(l == 0, np.where(odd, H2 + Q, H2), np.where(odd, H2 + l, L - l))
    # every frequency is evaluated exactly once
    assert np.array_equal(np.sort(np.concatenate([f0, f1])), np.arange(L))
    m = np.where(odd, np.where(l == 0, Q, H2 - l), l)
    pos = (m % M1) * 256 + m // M1
    assert np.array_equal(np.sort(pos), np.arange(H2))
    # each half-wave (32 lanes of one parity) stores one contiguous run
    for w in range(0, L // 2, 64):
        for par in (0, 1):
            p = pos[w + par:w + 64:2]
            d = np.diff(p)
            assert np.all(d == d[0]) and abs(d[0]) == 1 or (l[w] == 0 and par == 1)


@pytest.mark.parametrize("L", [8, 64, 32768, 65536])
def test_padded_spectrum_from_y(L):
    rng = np.random.default_rng(L + 7)
    X = rng.standard_normal(L) + 1j * rng.standard_normal(L)
    D = 0.37
    K = np.fft.ifft(X).real
    ref = np.fft.rfft(np.concatenate([K, np.zeros(L)])) + D        # bins 0..L
    m = np.arange(L // 2)
    xh = 0.5 * (X + np.conj(X[(-np.arange(L)) % L]))
    z = np.fft.ifft(_y_from_x(X)) * (L // 2) / L                    # K_2n + i K_2n+1
    F = np.fft.fft(z * np.exp(-2j * np.pi * m / L))
    p = L // 2 - 1 - m
    E = 0.5 * (F + np.conj(F[p]))
    O = (F - np.conj(F[p])) / 2j
    S = np.empty(L + 1, complex)
    S[2 * m + 1] = E + np.exp(-1j * np.pi * (2 * m + 1) / L) * O + D
    # the mirror bin as the row kernel writes it, from the same lane's values
    mirror = np.conj(E) + np.exp(-1j * np.pi * (2 * p + 1) / L) * np.conj(O) + D
    np.testing.assert_allclose(mirror, S[2 * p + 1], rtol=0, atol=1e-12)
    mm = np.arange(L // 2 + 1)
    S[2 * mm] = xh[mm % L] + D
    assert np.abs(S - ref).max() <= 1e-13 * np.abs(ref).max()
