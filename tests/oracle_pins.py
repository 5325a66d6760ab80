"""Pins for the CPU oracle: checks against what the paper and the mathematics fix.

Paper: "Elastic Selective Spectral Hybrids for Train-Once, Export-Many Budgeted
Inference" (ESSH).  Each pin takes a ``prefill`` callable with the signature of
``oracle.prefill`` so that the same checks can be run against deliberately
broken builds of the oracle (tests/test_oracle_mutants.py): every planted
mistake must make at least one pin fail.

Each pin returns (error, tolerance).  Errors are absolute errors normalised
by the largest magnitude of the expected result.
"""
from __future__ import annotations

import numpy as np
import scipy.signal

from oracle import reference


def _rand(seed, B, L, K, m, P, per_mode=False, rho=(0.80, 0.99)):
    rng = np.random.default_rng(seed)
    cs = (B, L, K, m) if per_mode else (B, L, K)
    return dict(
        v=rng.normal(size=(B, L, K, P)),
        delta=np.logaddexp(0.0, rng.normal(size=cs)),
        g_w=rng.uniform(0.05, 1.95, size=cs),
        g_r=rng.uniform(0.05, 1.95, size=cs),
        rho=rng.uniform(*rho, size=(K, m)),
        theta=rng.uniform(0.0, np.pi, size=(K, m)),
        c=rng.normal(0.0, 0.7, size=(K, m, 2)),
    )


def _nerr(a, b):
    scale = max(np.abs(b).max(), 1e-300)
    return float(np.abs(a - b).max() / scale)


def pin_closed_form_eq12(prefill, per_mode=False):
    """Sequential recurrence == closed-form double sum of App. B.4 Eq. 12 (zero initial state)."""
    x = _rand(11 + per_mode, B=2, L=48, K=3, m=3, P=5, per_mode=per_mode)
    y, _ = prefill(**x)
    yb = reference.brute_force(**x)
    return _nerr(y, yb), 1e-12


def pin_real_rotation_form(prefill):
    """Complex-mode oracle == the real 2xP damped rotation exactly as printed in Eq. 5, incl. states."""
    x = _rand(12, B=1, L=40, K=2, m=3, P=4)
    rng = np.random.default_rng(5)
    s0 = rng.normal(size=(1, 2, 3, 2, 4))
    y, st = prefill(**x, state_in=s0)
    yr, sr = reference.real_form(**x, state_in=s0)
    return max(_nerr(y, yr), _nerr(st, sr)), 1e-12


def pin_lti_fft(prefill, delta_const=0.0):
    """With a constant clock and unit gates the mixer is a causal convolution.

    Kernel psi(tau) = sum_j Re(c_j rho_j^tau e^{i theta_j tau}) (with rho
    replaced by rho e^{-delta} for a constant clock delta), evaluated by an
    rFFT of length 2L as in the ES-SSM FFT branch (ES-SSM App. C.2).
    """
    B, L, K, m, P = 2, 96, 3, 4, 6
    x = _rand(13, B, L, K, m, P)
    x["delta"] = np.full((B, L, K), delta_const)
    x["g_w"] = np.ones((B, L, K))
    x["g_r"] = np.ones((B, L, K))
    y, _ = prefill(**x)
    yf = np.zeros_like(y)
    n = 2 * L
    for k in range(K):
        psi = reference.lti_kernel(x["rho"][k], x["theta"][k], x["c"][k], L, delta_const)
        Hf = np.fft.rfft(psi, n)
        Vf = np.fft.rfft(x["v"][:, :, k, :], n, axis=1)
        yf[:, :, k, :] = np.fft.irfft(Vf * Hf[None, :, None], n, axis=1)[:, :L]
    return _nerr(y, yf), 1e-12


def pin_real_pole_iir(prefill):
    """One mode with a real pole (theta = 0 or pi, App. B.1) is a first-order IIR filter.

    y = lfilter([Re c], [1, -lam], v) with lam = +-rho e^{-delta}: a textbook
    special case computed by scipy.signal.lfilter.
    """
    B, L, K, m, P = 1, 200, 2, 1, 3
    x = _rand(14, B, L, K, m, P)
    d = 0.03
    x["delta"] = np.full((B, L, K), d)
    x["g_w"] = np.ones((B, L, K))
    x["g_r"] = np.ones((B, L, K))
    x["theta"] = np.array([[0.0], [np.pi]])
    y, _ = prefill(**x)
    err = 0.0
    for k, sign in ((0, 1.0), (1, -1.0)):
        lam = sign * x["rho"][k, 0] * np.exp(-d)
        ref = scipy.signal.lfilter([x["c"][k, 0, 0]], [1.0, -lam], x["v"][0, :, k, :], axis=0)
        err = max(err, _nerr(y[0, :, k, :], ref))
    return err, 1e-12


def pin_worked_example_eq15(prefill):
    """Three-position example of App. B.4 Eq. 15 (one mode, theta=0, kc=1, gates 1).

    z(3) = rho^2 e^{-Delta(3)} e^{-delta_pm} v(1), so the mixed difference over
    v(1) in {+1,-1} and Delta(2) in {delta+, delta-} is
    2 rho^2 e^{-Delta(3)} (e^{-delta+} - e^{-delta-}).
    """
    rho, d3, dp, dm = 0.93, 0.4, 1.7, 0.2
    vals = {}
    for v1 in (1.0, -1.0):
        for d2 in (dp, dm):
            x = dict(v=np.array([v1, 0.0, 0.0]).reshape(1, 3, 1, 1),
                     delta=np.array([0.8, d2, d3]).reshape(1, 3, 1),
                     g_w=np.ones((1, 3, 1)), g_r=np.ones((1, 3, 1)),
                     rho=np.array([[rho]]), theta=np.array([[0.0]]),
                     c=np.array([[[1.0, 0.0]]]))
            y, _ = prefill(**x)
            vals[(v1, d2)] = y[0, 2, 0, 0]
    mixed = vals[(1, dp)] - vals[(-1, dp)] - vals[(1, dm)] + vals[(-1, dm)]
    exact = 2 * rho ** 2 * np.exp(-d3) * (np.exp(-dp) - np.exp(-dm))
    single = vals[(1, dp)]
    return max(abs(mixed - exact) / abs(exact),
               abs(single - rho ** 2 * np.exp(-d3) * np.exp(-dp))), 1e-14


def pin_clock_shift_eq14(prefill):
    """Raising an intervening clock Delta(l) by delta scales what crosses l by e^{-delta} (Eq. 14).

    With v(s) = 0 for s >= l every contribution to y(t >= l) crosses position l,
    so those outputs scale by exactly e^{-delta}; outputs before l are unchanged.
    """
    B, L, K, m, P = 1, 60, 2, 3, 4
    x = _rand(15, B, L, K, m, P)
    ell, dd = 31, 0.37
    x["v"][:, ell:] = 0.0
    y0, _ = prefill(**x)
    x2 = dict(x)
    x2["delta"] = x["delta"].copy()
    x2["delta"][:, ell] += dd
    y1, _ = prefill(**x2)
    e1 = _nerr(y1[:, ell:], np.exp(-dd) * y0[:, ell:])
    e2 = _nerr(y1[:, :ell], y0[:, :ell])
    return max(e1, e2), 1e-13


def pin_state_contraction_eq16(prefill):
    """From a state h0 with no input, |h(t)| = rho^t e^{-q(t)} |h0| and the phase turns by theta t (Eq. 16)."""
    B, L, K, m, P = 1, 25, 2, 3, 4
    x = _rand(16, B, L, K, m, P)
    x["v"][:] = 0.0
    rng = np.random.default_rng(6)
    s0 = rng.normal(size=(B, K, m, 2, P))
    _, st = prefill(**x, state_in=s0)
    h0 = s0[:, :, :, 0] + 1j * s0[:, :, :, 1]
    q = x["delta"].sum(axis=1)                                     # [B, K]
    lam = x["rho"] ** L * np.exp(1j * x["theta"] * L)              # [K, m]
    expect = lam[None, :, :, None] * np.exp(-q)[:, :, None, None] * h0
    got = st[:, :, :, 0] + 1j * st[:, :, :, 1]
    return _nerr(got, expect), 1e-13


def pin_state_bound_eq17(prefill):
    """State norm bound of Eq. 17: ||H(t)||_F <= g_max V_max (1 - rho^t) / (1 - rho).

    (Eq. 17 uses g_max = 2 for the paper's (0,2) gates; the bound with the
    realised maximum write gate is the same argument.)  A sanity check.
    """
    B, L, K, m, P = 2, 64, 3, 2, 5
    x = _rand(17, B, L, K, m, P)
    _, st = prefill(**x)
    gmax = x["g_w"].max()
    vmax = np.linalg.norm(x["v"], axis=-1).max()
    norms = np.sqrt((st ** 2).sum(axis=(3, 4)))                     # [B, K, m]
    bound = gmax * vmax * (1 - x["rho"] ** L) / (1 - x["rho"])      # [K, m]
    ratio = float((norms / bound[None]).max())
    return max(0.0, ratio - 1.0), 0.0


def pin_chunked_equals_sequential(prefill, Lc=16, L=53, per_mode=False):
    """The chunk decomposition (Sec. 4.3, from Eq. 6) equals the sequential scan, ragged tail included."""
    x = _rand(18 + Lc + per_mode, B=2, L=L, K=3, m=4, P=6, per_mode=per_mode)
    rng = np.random.default_rng(7)
    s0 = rng.normal(size=(2, 3, 4, 2, 6))
    y, st = prefill(**x, state_in=s0)
    yc, sc = reference.chunked(**x, Lc=Lc, state_in=s0)
    return max(_nerr(y, yc), _nerr(st, sc)), 1e-12


def pin_zero_lag_recurrence(prefill, per_mode=False):
    """Zero-lag correction (Eq. 24) against the equivalent J recurrence of App. C.3.

    The oracle subtracts a g_r g_w kc v from the core readout; the reference
    never forms the core readout: it runs J(t) = A J(t-1) + (1-a) b(t) + a A b(t-1)
    and reads J directly.  State in and out included; a ~ U(0, 1) around the
    paper's initial value 1/2.
    """
    B, L, K, m, P = 2, 37, 3, 4, 5
    x = _rand(31, B, L, K, m, P, per_mode=per_mode)
    rng = np.random.default_rng(32)
    zl = rng.uniform(0.0, 1.0, size=(K, m))
    s0 = rng.normal(0, 1.0, size=(B, K, m, 2, P))
    y, st = prefill(**x, zl=zl, state_in=s0)
    yr, sr = reference.zero_lag_jrec(**x, zl=zl, state_in=s0)
    return max(_nerr(y, yr), _nerr(st, sr)), 1e-12


def pin_zero_lag_lti_fft(prefill):
    """With a constant clock and unit gates the corrected mixer is a causal
    convolution whose lag-zero tap is psi(0) - sum_j a_j kc_j (App. C.3: the
    correction changes only the lag-zero coefficient); evaluated by rFFT."""
    B, L, K, m, P = 2, 80, 3, 4, 6
    x = _rand(33, B, L, K, m, P)
    x["delta"] = np.zeros((B, L, K))
    x["g_w"] = np.ones((B, L, K))
    x["g_r"] = np.ones((B, L, K))
    zl = np.random.default_rng(34).uniform(0.0, 1.0, size=(K, m))
    y, _ = prefill(**x, zl=zl)
    yf = np.zeros_like(y)
    n = 2 * L
    for k in range(K):
        phi = reference.lti_kernel(x["rho"][k], x["theta"][k], x["c"][k], L, 0.0)
        phi[0] -= float(np.sum(zl[k] * x["c"][k][:, 0]))
        Hf = np.fft.rfft(phi, n)
        Vf = np.fft.rfft(x["v"][:, :, k, :], n, axis=1)
        yf[:, :, k, :] = np.fft.irfft(Vf * Hf[None, :, None], n, axis=1)[:, :L]
    return _nerr(y, yf), 1e-12


ALL_PINS = [
    ("closed_form_eq12", pin_closed_form_eq12, {}),
    ("closed_form_eq12_per_mode", pin_closed_form_eq12, {"per_mode": True}),
    ("real_rotation_form_eq5", pin_real_rotation_form, {}),
    ("lti_fft", pin_lti_fft, {}),
    ("lti_fft_const_clock", pin_lti_fft, {"delta_const": 0.05}),
    ("real_pole_iir", pin_real_pole_iir, {}),
    ("worked_example_eq15", pin_worked_example_eq15, {}),
    ("clock_shift_eq14", pin_clock_shift_eq14, {}),
    ("state_contraction_eq16", pin_state_contraction_eq16, {}),
    ("state_bound_eq17", pin_state_bound_eq17, {}),
    ("chunked_eq6_Lc16", pin_chunked_equals_sequential, {"Lc": 16}),
    ("chunked_eq6_Lc8_per_mode", pin_chunked_equals_sequential, {"Lc": 8, "per_mode": True}),
    ("zero_lag_recurrence_eq24", pin_zero_lag_recurrence, {}),
    ("zero_lag_recurrence_eq24_per_mode", pin_zero_lag_recurrence, {"per_mode": True}),
    ("zero_lag_lti_fft", pin_zero_lag_lti_fft, {}),
]
