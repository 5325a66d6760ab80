"""NumPy restatements of the selective mixer core -- TEST INFRASTRUCTURE.

Each function computes the same result as the sequential C oracle by a
different route taken from the paper ("Elastic Selective Spectral Hybrids for
Train-Once, Export-Many Budgeted Inference"), so that agreement between them
pins the oracle.  All arithmetic is float64.  Shapes as in ``oracle.prefill``.
Mode index j, channel k, value coordinate p; positions t are 0-based here
(the paper counts from 1).
"""
from __future__ import annotations

import numpy as np


def _ctrl(x, m):
    """Broadcast per-channel controls [B,L,K] to per-mode [B,L,K,m]."""
    x = np.asarray(x, np.float64)
    return x if x.ndim == 4 else np.repeat(x[..., None], m, axis=-1)


def brute_force(v, delta, g_w, g_r, rho, theta, c, K_T=None):
    """Closed-form expansion of the selective recurrence from a zero state (App. B.4, Eq. 12).

    z_k(t) = sum_{s<=t} sum_j g_r,j(t) g_w,j(s) exp(-(q_j(t)-q_j(s))) psi_j(t-s) v_k(s)
    with q_j(t) the running sum of the clock up to and including t, and
    psi_j(tau) = rho_j^tau (kc_j cos(theta_j tau) - ks_j sin(theta_j tau)).
    O(L^2) per channel; only for small inputs.
    """
    v = np.asarray(v, np.float64)
    B, L, K, P = v.shape
    m = np.shape(rho)[1]
    K_T = K if K_T is None else K_T
    dl, gw, gr = _ctrl(delta, m), _ctrl(g_w, m), _ctrl(g_r, m)
    y = np.zeros_like(v)
    tau = np.arange(L)
    for b in range(B):
        for k in range(K_T):
            for j in range(m):
                r, th = float(rho[k][j]), float(theta[k][j])
                kc, ks = float(c[k][j][0]), float(c[k][j][1])
                psi = r ** tau * (kc * np.cos(th * tau) - ks * np.sin(th * tau))
                q = np.cumsum(dl[b, :, k, j])
                for t in range(L):
                    s = np.arange(t + 1)
                    coef = gr[b, t, k, j] * gw[b, s, k, j] * np.exp(-(q[t] - q[s])) * psi[t - s]
                    y[b, t, k] += coef @ v[b, s, k]
    return y


def real_form(v, delta, g_w, g_r, rho, theta, c, K_T=None, state_in=None):
    """The recurrence exactly as printed in Eq. 5: a real 2xP state per mode.

    H(t) = rho exp(-delta(t)) R(theta) H(t-1) + g_w(t) e1 v(t)^T,
    z(t) = sum_j g_r,j(t) H_j(t)^T kappa_j,  kappa = (kc, -ks),
    R(theta) = [[cos, -sin], [sin, cos]].  Returns (y, state [B,K,m,2,P]).
    """
    v = np.asarray(v, np.float64)
    B, L, K, P = v.shape
    m = np.shape(rho)[1]
    K_T = K if K_T is None else K_T
    dl, gw, gr = _ctrl(delta, m), _ctrl(g_w, m), _ctrl(g_r, m)
    y = np.zeros_like(v)
    st = np.zeros((B, K, m, 2, P))
    for b in range(B):
        for k in range(K_T):
            H = np.zeros((m, 2, P)) if state_in is None else np.array(state_in[b, k], np.float64)
            for t in range(L):
                for j in range(m):
                    th = float(theta[k][j])
                    R = np.array([[np.cos(th), -np.sin(th)], [np.sin(th), np.cos(th)]])
                    A = float(rho[k][j]) * np.exp(-dl[b, t, k, j]) * R
                    H[j] = A @ H[j]
                    H[j, 0] += gw[b, t, k, j] * v[b, t, k]
                    kappa = np.array([c[k][j][0], -c[k][j][1]], np.float64)
                    y[b, t, k] += gr[b, t, k, j] * (kappa @ H[j])
            st[b, k] = H
    return y, st


def zero_lag_jrec(v, delta, g_w, g_r, rho, theta, c, zl, K_T=None, state_in=None):
    """The zero-lag corrected output (App. C.3, Eq. 24) by its equivalent recurrence.

    App. C.3 rewrites the correction without touching the readout: with
    b(t) = g_w(t) e1 v(t)^T and J(t) = H(t) - a b(t),
      J(t) = A(t) J(t-1) + (1 - a) b(t) + a A(t) b(t-1),    b(-1) = 0,
    and the corrected output is z(t) = sum_j g_r,j(t) J_j(t)^T kappa_j.  Real
    2xP form as printed (A = rho e^{-delta} R(theta), kappa = (kc, -ks)).
    Returns (z, state) with state = H(L-1) = J(L-1) + a b(L-1).
    """
    v = np.asarray(v, np.float64)
    B, L, K, P = v.shape
    m = np.shape(rho)[1]
    K_T = K if K_T is None else K_T
    dl, gw, gr = _ctrl(delta, m), _ctrl(g_w, m), _ctrl(g_r, m)
    y = np.zeros_like(v)
    st = np.zeros((B, K, m, 2, P))
    for b in range(B):
        for k in range(K_T):
            J = np.zeros((m, 2, P)) if state_in is None else np.array(state_in[b, k], np.float64)
            bprev = np.zeros((m, 2, P))
            for t in range(L):
                for j in range(m):
                    a = float(zl[k][j])
                    th = float(theta[k][j])
                    R = np.array([[np.cos(th), -np.sin(th)], [np.sin(th), np.cos(th)]])
                    A = float(rho[k][j]) * np.exp(-dl[b, t, k, j]) * R
                    bt = np.zeros((2, P))
                    bt[0] = gw[b, t, k, j] * v[b, t, k]
                    J[j] = A @ J[j] + (1.0 - a) * bt + a * (A @ bprev[j])
                    bprev[j] = bt
                    kappa = np.array([c[k][j][0], -c[k][j][1]], np.float64)
                    y[b, t, k] += gr[b, t, k, j] * (kappa @ J[j])
            for j in range(m):
                st[b, k, j] = J[j] + float(zl[k][j]) * bprev[j]
    return y, st


def chunked(v, delta, g_w, g_r, rho, theta, c, Lc, K_T=None, state_in=None):
    """Chunk decomposition of the scan (Sec. 4.3), derived from the transition product Eq. 6.

    For a chunk [t0, t1) of n positions with chunk-local inclusive clock sums
    qh(t) = sum_{l=t0..t} delta(l) and constant poles lam_j = rho_j e^{i theta_j}:
      intra:  y(t) += sum_{t0<=s<=t} sum_j g_r(t) g_w(s) e^{-(qh(t)-qh(s))} Re(c_j lam_j^{t-s}) v(s)
      carry:  y(t) += sum_j g_r(t) e^{-qh(t)} Re(c_j lam_j^{t-t0+1} h_j)
      state:  h_j <- lam_j^n e^{-qh(t1-1)} h_j + sum_s lam_j^{t1-1-s} e^{-(qh(t1-1)-qh(s))} g_w(s) v(s)
    where h_j is the complex mode state entering the chunk.  A ragged last
    chunk (n < Lc) is allowed.  Returns (y, state [B,K,m,2,P]).
    """
    v = np.asarray(v, np.float64)
    B, L, K, P = v.shape
    m = np.shape(rho)[1]
    K_T = K if K_T is None else K_T
    dl, gw, gr = _ctrl(delta, m), _ctrl(g_w, m), _ctrl(g_r, m)
    y = np.zeros_like(v)
    st = np.zeros((B, K, m, 2, P))
    for b in range(B):
        for k in range(K_T):
            lam = np.asarray(rho[k], np.float64) * np.exp(1j * np.asarray(theta[k], np.float64))
            cc = np.asarray(c[k][:, 0], np.float64) + 1j * np.asarray(c[k][:, 1], np.float64)
            if state_in is None:
                h = np.zeros((m, P), complex)
            else:
                h = state_in[b, k, :, 0] + 1j * state_in[b, k, :, 1]
            for t0 in range(0, L, Lc):
                t1 = min(t0 + Lc, L)
                n = t1 - t0
                V = v[b, t0:t1, k]                        # [n, P]
                r = np.arange(n)
                for j in range(m):
                    qh = np.cumsum(dl[b, t0:t1, k, j])     # inclusive, chunk-local
                    lag = r[:, None] - r[None, :]
                    pw = lam[j] ** np.maximum(lag, 0)
                    G = np.where(lag >= 0,
                                 gr[b, t0:t1, k, j][:, None] * gw[b, t0:t1, k, j][None, :]
                                 * np.exp(-(qh[:, None] - qh[None, :])) * np.real(cc[j] * pw),
                                 0.0)
                    y[b, t0:t1, k] += G @ V
                    carry = (gr[b, t0:t1, k, j] * np.exp(-qh))[:, None] * np.real(
                        cc[j] * lam[j] ** (r + 1)[:, None] * h[j][None, :])
                    y[b, t0:t1, k] += carry
                    w = lam[j] ** (n - 1 - r) * np.exp(-(qh[-1] - qh)) * gw[b, t0:t1, k, j]
                    h[j] = lam[j] ** n * np.exp(-qh[-1]) * h[j] + w @ V
            st[b, k, :, 0] = h.real
            st[b, k, :, 1] = h.imag
    return y, st


def lti_kernel(rho, theta, c, L, delta_const=0.0):
    """Impulse response of one channel with constant clock and unit gates.

    psi(tau) = sum_j Re(c_j (rho_j e^{-delta} e^{i theta_j})^tau), tau = 0..L-1
    (App. B.1 modal form; Eq. 4 with the clock folded into the decay).
    rho, theta [m], c [m,2].
    """
    tau = np.arange(L)[:, None]
    lam = np.asarray(rho, np.float64) * np.exp(-delta_const) * np.exp(1j * np.asarray(theta, np.float64))
    cc = np.asarray(c, np.float64)[:, 0] + 1j * np.asarray(c, np.float64)[:, 1]
    return np.real(cc[None, :] * lam[None, :] ** tau).sum(axis=1)
