"""Pins of the Hankel filter bank and its matrix-pencil mode fit (selective_spectral_ssm_amd/
modefit.py), CPU only: Eq. 10 against numerical integration, the sign-change count of App. B.2,
the statistics App. B.7 / App. C.1.1 print for L = 2048 and m = 8 (tests/golden/b7_mode_fit.txt),
Eq. 21 against quadrature over lambda, exact recovery of a signal made of m damped modes, and
the fitted tables run through the oracle's recurrence as an impulse response."""
import math
import os

import numpy as np
import pytest
from scipy import integrate

from selective_spectral_ssm_amd import modefit

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "b7_mode_fit.txt")


@pytest.fixture(scope="module")
def fit2048():
    return modefit.fit_mode_tables(32, 8, L=2048)


def _stated():
    out = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, val, digits = line.split()
        out[name] = (float(val), int(digits))
    return out


def _rounds_to(x, val, digits):
    """x printed with `digits` significant digits reads val"""
    return float(f"{x:.{digits - 1}e}") == val


def test_eq10_against_integration():
    Z = modefit.hankel_matrix(9)
    for s, t in ((1, 1), (1, 5), (3, 7), (9, 9), (2, 8)):
        val, _ = integrate.quad(lambda lam: (1 - lam) ** 2 * lam ** (s + t - 2), 0.0, 1.0, epsabs=1e-15, epsrel=1e-13)
        assert abs(Z[s - 1, t - 1] - val) <= 1e-13 * max(1.0, val)


def test_sign_changes_of_the_filters():
    sigma, phi = modefit.hankel_filters(2048)
    assert np.all(np.diff(sigma[:40]) < 0)
    for k in range(12):
        assert modefit.sign_changes(phi[:, k]) == k


def test_stated_statistics(fit2048):
    st = _stated()
    sigma, err = fit2048["sigma"], fit2048["fit_err"]
    tr = sigma.sum()
    assert abs(tr - np.trace(modefit.hankel_matrix(2048))) <= 1e-12 * tr
    assert _rounds_to(sigma[8] / sigma[0], *st["sigma9_over_sigma1"])
    assert _rounds_to(sigma[8:].sum() / tr, *st["tail_beyond_8_over_trace"])
    assert _rounds_to(err[:8].max(), *st["max_fit_error_first_8_channels"])
    bound = st["projection_fit_error_over_trace_bound"][0]
    for K in (8, 16, 24, 32):
        assert modefit.projection_fit_error(sigma, err, K) / tr < bound
    # more oscillatory channels fit worse with the same mode budget
    assert err[8:].min() > err[:8].max()


def test_eq21_against_quadrature():
    """E_K^(m) = E_lambda || mu(lambda) - sum_k <mu, phi_k> phi_hat_k ||^2 equals the projection
    tail plus the eigenvalue-weighted fit errors (tiny L, integrated over lambda)."""
    L, K, m = 48, 4, 3
    sigma, phi = modefit.hankel_filters(L)
    fits, errs = [], []
    for k in range(K):
        r, th, c, e = modefit.matrix_pencil_fit(phi[:, k], m, pencil=16)
        fits.append(modefit.modal_response(r, th, c, L))
        errs.append(e)
    fits = np.stack(fits, axis=1)                      # [L, K]
    t = np.arange(L)

    def integrand(lam):
        mu = (1 - lam) * lam ** t
        res = mu - fits @ (phi[:, :K].T @ mu)
        return float(res @ res)

    val, _ = integrate.quad(integrand, 0.0, 1.0, limit=400, epsabs=1e-14, epsrel=1e-10)
    want = modefit.projection_fit_error(sigma, np.array(errs), K)
    assert abs(val - want) <= 1e-7 * want


def test_pencil_recovers_exact_modes():
    """A real signal of m0 rotating modes has the 2 m0 poles lambda_j and their conjugates; a fit
    with m = 2 m0 modes finds exactly those and reproduces the signal."""
    rng = np.random.default_rng(3)
    m0, N = 3, 400
    rho = rng.uniform(0.9, 0.995, m0)
    theta = rng.uniform(0.2, 3.0, m0)
    c = rng.normal(size=m0) + 1j * rng.normal(size=m0)
    x = modefit.modal_response(rho, theta, c, N)
    r, th, cc, e = modefit.matrix_pencil_fit(x, 2 * m0, pencil=100)
    assert e < 1e-9
    got = sorted(zip(np.round(th, 6), np.round(r, 9)))
    want = sorted(zip(np.round(np.concatenate([theta, -theta]), 6), np.round(np.concatenate([rho, rho]), 9)))
    for (a1, b1), (a2, b2) in zip(got, want):
        assert abs(a1 - a2) < 1e-5 and abs(b1 - b2) < 1e-8


def test_fitted_tables_are_the_recurrence_impulse_response(fit2048):
    """Unit gates, zero clock, an impulse at position 0: the oracle's recurrence outputs the
    fitted response sum_j Re(c_j lambda_j^tau), and that is within the fit error of phi_k."""
    import oracle
    K, m, n = 8, 8, 2048
    _, phi = modefit.hankel_filters(n)
    rho, theta, c = (fit2048[k][:K].astype(np.float64) for k in ("rho", "theta", "c"))
    v = np.zeros((1, n, K, 1))
    v[0, 0] = 1.0
    zero = np.zeros((1, n, K))
    y, _ = oracle.prefill(v, zero, zero + 1.0, zero + 1.0, rho, theta, c)
    for k in range(K):
        want = modefit.modal_response(rho[k], theta[k], c[k, :, 0] + 1j * c[k, :, 1], n)
        assert np.allclose(y[0, :, k, 0], want, rtol=1e-9, atol=1e-12)
        rel = np.linalg.norm(y[0, :, k, 0] - phi[:, k]) / np.linalg.norm(phi[:, k])
        assert rel <= fit2048["fit_err"][k] + 1e-5       # float32 tables
