"""Initial mode tables: the Hankel filter bank and its matrix-pencil mode fit (host side).

ESSH paper (Elastic Selective Spectral Hybrids for Train-Once, Export-Many Budgeted
Inference), App. B.3 Eq. 10, App. B.2, App. B.7 and App. C.1.1:

  * Z_st = 2 / ((s + t - 1)(s + t)(s + t + 1)), s, t = 1..L (Eq. 10), the second moment of the
    (1 - lambda)-weighted power family under lambda ~ Unif[0, 1]; its eigenvectors phi_k,
    ordered by decreasing eigenvalue sigma_k, are the spectral channels' filters;
  * each filter (length L) is fitted by a matrix pencil: the Hankel data matrix of pencil
    parameter 512, a rank-m truncated SVD, the m poles as eigenvalues of the shifted pencil of
    the retained right singular vectors, each pole one damped mode (conjugate poles take
    separate modes), magnitudes clipped to stable decays, then the complex readout
    coefficients by least squares;
  * the fitted response of channel k is phi_hat_k(tau) = sum_j Re(c_j lambda_j^tau), tau = t - 1,
    the modal response the recurrence realizes with unit gates and zero clock.

The tables (rho, theta, c) are float32 in the layout the library takes: rho, theta [K, m],
c [K, m, 2] (real, imaginary).  Everything here is float64 NumPy on the host; it is an
initializer, not part of the GPU path.
"""
from __future__ import annotations

import numpy as np

PENCIL = 512            # pencil parameter of the fit (App. C.1.1)
RHO_MAX = 1.0 - 1e-6    # stable-decay clip of the fitted pole magnitudes


def hankel_matrix(L: int) -> np.ndarray:
    """Z of Eq. 10, [L, L]."""
    s = np.arange(1, L + 1, dtype=np.float64)
    n = s[:, None] + s[None, :]
    return 2.0 / ((n - 1.0) * n * (n + 1.0))


def hankel_filters(L: int):
    """(sigma [L] decreasing, phi [L, L] with phi[:, k] the filter of channel k + 1), each
    filter signed so that its first entry is positive."""
    w, v = np.linalg.eigh(hankel_matrix(L))
    w, v = w[::-1].copy(), v[:, ::-1].copy()
    v *= np.where(v[0] < 0, -1.0, 1.0)[None, :]
    return w, v


def sign_changes(x: np.ndarray, rel_tol: float = 1e-12) -> int:
    """Sign changes of x with (near-)zero entries left out (App. B.2)."""
    x = x[np.abs(x) > rel_tol * np.abs(x).max()]
    return int(np.count_nonzero(np.signbit(x[1:]) != np.signbit(x[:-1])))


def modal_response(rho, theta, c, n: int) -> np.ndarray:
    """sum_j Re(c_j lambda_j^tau) for tau = 0..n-1; c complex [m]."""
    tau = np.arange(n)[:, None]
    z = rho[None, :] ** tau * np.exp(1j * theta[None, :] * tau)
    return (z * c[None, :]).real.sum(axis=1)


def matrix_pencil_fit(x: np.ndarray, m: int, pencil: int = PENCIL, rho_max: float = RHO_MAX):
    """Fit x[tau] ~ sum_j Re(c_j lambda_j^tau) with m modes.  Returns (rho [m], theta [m],
    c [m] complex, relative error ||x - fit|| / ||x||)."""
    x = np.asarray(x, dtype=np.float64)
    N = x.shape[0]
    lp = min(pencil, N - 1)
    Y = np.lib.stride_tricks.sliding_window_view(x, lp + 1)          # [N - lp, lp + 1] Hankel
    _, _, vh = np.linalg.svd(Y, full_matrices=False)
    vm = vh[:m].conj().T                                             # [lp + 1, m]
    poles = np.linalg.eigvals(np.linalg.pinv(vm[:-1]) @ vm[1:])
    rho = np.minimum(np.abs(poles), rho_max)
    theta = np.angle(poles)
    # readout coefficients: real least squares in (Re c, Im c)
    tau = np.arange(N)[:, None]
    z = rho[None, :] ** tau * np.exp(1j * theta[None, :] * tau)
    A = np.concatenate([z.real, -z.imag], axis=1)
    coef, *_ = np.linalg.lstsq(A, x, rcond=None)
    c = coef[:m] + 1j * coef[m:]
    err = float(np.linalg.norm(x - A @ coef) / np.linalg.norm(x))
    return rho, theta, c, err


def fit_mode_tables(K: int, m: int, L: int = 2048):
    """Mode tables of the first K channels fitted with m modes each.

    Returns dict(rho [K, m] f32, theta [K, m] f32, c [K, m, 2] f32, fit_err [K], sigma [L])."""
    sigma, phi = hankel_filters(L)
    rho = np.empty((K, m), np.float32)
    theta = np.empty((K, m), np.float32)
    c = np.empty((K, m, 2), np.float32)
    err = np.empty(K)
    for k in range(K):
        r, th, cc, e = matrix_pencil_fit(phi[:, k], m)
        rho[k], theta[k] = r, th
        c[k, :, 0], c[k, :, 1] = cc.real, cc.imag
        err[k] = e
    return dict(rho=rho, theta=theta, c=c, fit_err=err, sigma=sigma)


def projection_fit_error(sigma: np.ndarray, fit_err: np.ndarray, K: int) -> float:
    """Eq. 21: the Hankel projection tail beyond channel K plus the fit errors of the retained
    channels weighted by their eigenvalues (divide by trace Z = sum(sigma) for the relative
    figure)."""
    return float(sigma[K:].sum() + np.sum(sigma[:K] * fit_err[:K] ** 2))
