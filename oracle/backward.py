"""Reverse-mode gradients of the prefill -- TEST INFRASTRUCTURE (oracle extension).

Only ``tests/`` may use this module; the product path never imports it.  The forward
computation is the recurrence of the paper "Elastic Selective Spectral Hybrids for Train-Once,
Export-Many Budgeted Inference", Sec. 4.1 Eq. 5 in the complex form of App. B.1, the readout
of Eq. 9 and the optional zero-lag correction of App. C.3 Eq. 24, with controls per mode
(Eq. 5, App. C.2) or per channel (the same value broadcast over the modes):

    lambda_j(t) = rho_j e^{-delta_j(t)} e^{i theta_j}
    h_j(t)      = lambda_j(t) h_j(t-1) + g_w,j(t) v(t)                  h_j(-1) = state_in
    y(t)        = sum_j g_r,j(t) [Re(c_j h_j(t)) - a_j Re(c_j) g_w,j(t) v(t)]

For a loss with dL/dy = dy and dL/dh(L-1) = dstate_out, the adjoint of mode j's state,
abar_j(t) = dL/dRe h_j(t) + i dL/dIm h_j(t), satisfies

    abar_j(t) = g_r,j(t) dy(t) conj(c_j) + conj(lambda_j(t+1)) abar_j(t+1),
    abar_j(L-1) additionally receives dstate_out,   dstate_in = conj(lambda_j(0)) abar_j(0),

and the gradient of any quantity x that enters step t is Re(conj(abar_j(t)) dh_j(t)/dx), summed
over value columns p (and batch rows, positions for the mode tables).  Each step below writes
out one term of these sums; nothing is blocked or reordered.  Per-channel controls are
handled by broadcasting them over the modes and summing the per-mode gradients (chain rule of
the broadcast).  Everything is float64, a loop over positions vectorized over (b, k, j, p).

Layouts as the C oracle: v, dy [B, L, K, P]; delta, g_w, g_r [B, L, K] or [B, L, K, m];
rho, theta [K, m]; c [K, m, 2]; zl [K, m] or None; state [B, K, m, 2, P].  Gradients have the
layout of their inputs; channels k >= K_T receive zero.
"""
from __future__ import annotations

import numpy as np


def prefill_backward(v, delta, g_w, g_r, rho, theta, c, dy, K_T=None, state_in=None, dstate_out=None,
                     zl=None):
    """Returns dict(dv, ddelta, dg_w, dg_r, drho, dtheta, dc, dstate_in, dzl (None without zl),
    y, state_out) -- the last two are the forward results of the same pass."""
    v = np.asarray(v, np.float64)
    B, L, K, P = v.shape
    m = np.shape(rho)[1]
    per_mode = np.ndim(delta) == 4
    kt = K if K_T is None else int(K_T)
    sl = slice(0, kt)

    def modes(x):                                 # controls as [B, L, kt, m]
        x = np.asarray(x, np.float64)[:, :, sl]
        return x if per_mode else np.repeat(x[..., None], m, axis=-1)

    dl, gw, gr = modes(delta), modes(g_w), modes(g_r)
    vv = v[:, :, sl]                                                                      # [B, L, kt, P]
    dyy = np.asarray(dy, np.float64)[:, :, sl]
    rr, th = np.asarray(rho, np.float64)[sl], np.asarray(theta, np.float64)[sl]          # [kt, m]
    cc = np.asarray(c, np.float64)[sl, :, 0] + 1j * np.asarray(c, np.float64)[sl, :, 1]
    aa = np.zeros((kt, m)) if zl is None else np.asarray(zl, np.float64)[sl]
    pole = rr * np.exp(1j * th)

    def lam(t):                                   # lambda_j(t), [B, kt, m]
        return pole[None] * np.exp(-dl[:, t])

    # forward: every state, [L, B, kt, m, P]
    h = np.zeros((L, B, kt, m, P), np.complex128)
    if state_in is None:
        h_init = np.zeros((B, kt, m, P), np.complex128)
    else:
        s = np.asarray(state_in, np.float64)[:, sl]
        h_init = s[:, :, :, 0] + 1j * s[:, :, :, 1]
    hp = h_init
    for t in range(L):
        hp = lam(t)[..., None] * hp + gw[:, t, :, :, None] * vv[:, t, :, None, :]
        h[t] = hp
    y = np.zeros((B, L, K, P))
    for t in range(L):
        core = np.sum(gr[:, t, :, :, None] * (cc[None, :, :, None] * h[t]).real, axis=2)
        lag0 = np.sum(gr[:, t] * gw[:, t] * (aa * cc.real)[None], axis=2)              # [B, kt]
        y[:, t, sl] = core - lag0[..., None] * vv[:, t]

    # backward, positions L-1 .. 0
    ab = np.zeros((B, kt, m, P), np.complex128)
    if dstate_out is not None:
        so = np.asarray(dstate_out, np.float64)[:, sl]
        ab = ab + so[:, :, :, 0] + 1j * so[:, :, :, 1]
    dv = np.zeros((B, L, K, P))
    ddl = np.zeros((B, L, kt, m))
    dgw = np.zeros((B, L, kt, m))
    dgr = np.zeros((B, L, kt, m))
    drho = np.zeros((K, m))
    dtheta = np.zeros((K, m))
    dc = np.zeros((K, m, 2))
    dzl = np.zeros((K, m))
    for t in range(L - 1, -1, -1):
        dyt, vt = dyy[:, t], vv[:, t]                                                     # [B, kt, P]
        grt, gwt = gr[:, t], gw[:, t]                                                     # [B, kt, m]
        vdy = np.sum(vt * dyt, axis=-1)                                                   # [B, kt]
        # readout: y(t) depends on h_j(t) through g_r,j(t) Re(c_j h_j(t))
        ab = ab + (grt[..., None] * dyt[:, :, None, :]) * np.conj(cc)[None, :, :, None]
        dgr[:, t] = np.sum(dyt[:, :, None, :] * (cc[None, :, :, None] * h[t]).real, axis=-1)
        gdy = grt[..., None] * dyt[:, :, None, :]                                         # [B, kt, m, P]
        dc[sl, :, 0] += np.sum(gdy * h[t].real, axis=(0, 3))
        dc[sl, :, 1] -= np.sum(gdy * h[t].imag, axis=(0, 3))
        # zero-lag term -g_r,j g_w,j a_j Re(c_j) v(t)
        za = (aa * cc.real)[None]                                                         # [1, kt, m]
        dv[:, t, sl] = -np.sum(grt * gwt * za, axis=2)[..., None] * dyt
        dgr[:, t] -= gwt * za * vdy[..., None]
        dgw[:, t] = -grt * za * vdy[..., None]
        dzl[sl] -= np.sum(grt * gwt * vdy[..., None], axis=0) * cc.real
        dc[sl, :, 0] -= np.sum(grt * gwt * vdy[..., None], axis=0) * aa
        # injection g_w,j(t) v(t) into the real part of mode j's state
        dv[:, t, sl] += np.sum(gwt[..., None] * ab.real, axis=2)
        dgw[:, t] += np.sum(vt[:, :, None, :] * ab.real, axis=-1)
        # transition lambda_j(t) h_j(t-1): d/d delta = -lambda h, d/d rho = lambda h / rho,
        # d/d theta = i lambda h
        hprev = h[t - 1] if t > 0 else h_init
        inner = np.conj(ab) * (lam(t)[..., None] * hprev)                                 # [B, kt, m, P]
        ddl[:, t] = -np.sum(inner.real, axis=-1)
        drho[sl] += np.sum(inner.real, axis=(0, 3)) / rr
        dtheta[sl] += np.sum((1j * inner).real, axis=(0, 3))
        ab = np.conj(lam(t))[..., None] * ab
    dstate_in = np.zeros((B, K, m, 2, P))
    dstate_in[:, sl, :, 0] = ab.real
    dstate_in[:, sl, :, 1] = ab.imag
    state_out = np.zeros((B, K, m, 2, P))
    state_out[:, sl, :, 0] = h[L - 1].real if L else h_init.real
    state_out[:, sl, :, 1] = h[L - 1].imag if L else h_init.imag

    def ctrl_grad(g):                             # back to the controls' own layout
        out = np.zeros((B, L, K, m) if per_mode else (B, L, K))
        out[:, :, sl] = g if per_mode else g.sum(axis=-1)
        return out

    return dict(dv=dv, ddelta=ctrl_grad(ddl), dg_w=ctrl_grad(dgw), dg_r=ctrl_grad(dgr), drho=drho,
                dtheta=dtheta, dc=dc, dstate_in=dstate_in, dzl=None if zl is None else dzl, y=y,
                state_out=state_out)
