"""Fused decode step with its projections -- TEST INFRASTRUCTURE (oracle extension).

Only ``tests/`` (and the CPU baseline of ``bench.py``) may use this module; the product path
never imports it.  It follows the paper "Elastic Selective Spectral Hybrids for Train-Once,
Export-Many Budgeted Inference":

  * App. C.2, "Projections, gates, and clock": v0_k = W_in_k u, the channel-local blend of
    Eq. 23, v_k = (1 - beta_k) v0_k + beta_k v0_k / sqrt(P^-1 ||v0_k||^2 + eps), and per
    (channel, mode) the affine rows giving the write gate 2 sigmoid(.), the read gate
    2 sigmoid(.) and the clock increment softplus(.);
  * Sec. 4.1, Eq. 5 with per-mode controls, and App. C.3, Eq. 24 (zero-lag correction): one
    step of the mode recurrence and its readout z_k, by the C oracle's decode step;
  * App. C.4, "Channel aggregation and the complete computation": the z_k of the first K_T
    channels, concatenated, times the first K_T P columns of W_out, scaled by K_T^-1/2.

Weights and inputs are real arrays (already upcast from bf16 where the GPU reads bf16); all
arithmetic is float64.  Layouts (d = model width):
  u [NL, B, d]; w_in [NL, K, P, d] (row (k, p) of W_in); beta [NL, K];
  w_ctl [NL, K, m, 3, d] and b_ctl [NL, K, m, 3] (rows: write gate, read gate, clock);
  rho, theta [NL, K, m]; c [NL, K, m, 2]; zl [NL, K, m] or None;
  w_out [NL, d, K, P] (row o of W_out, columns grouped by channel); state [NL, B, K, m, 2, P].
"""
from __future__ import annotations

import numpy as np


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    # log(1 + e^x), written so that it neither overflows nor loses precision for large |x|
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def channel_values(u, w_in, beta, eps, K_T):
    """App. C.2: v0_k = W_in_k u, then Eq. 23's blend with channel k's own statistic.
    u [B, d]; w_in [K, P, d]; beta [K]  ->  v [B, K_T, P]."""
    v0 = np.einsum("kpd,bd->bkp", w_in[:K_T], u)
    ms = np.mean(v0 * v0, axis=-1, keepdims=True)          # P^-1 ||v0_k||^2, channel k only
    bt = beta[:K_T][None, :, None]
    return (1.0 - bt) * v0 + bt * v0 / np.sqrt(ms + eps)


def controls(u, w_ctl, b_ctl, K_T):
    """App. C.2: per (channel, mode) write gate, read gate and clock increment.
    u [B, d]; w_ctl [K, m, 3, d]; b_ctl [K, m, 3]  ->  three arrays [B, K_T, m]."""
    a = np.einsum("kmsd,bd->bkms", w_ctl[:K_T], u) + b_ctl[:K_T][None]
    return 2.0 * _sigmoid(a[..., 0]), 2.0 * _sigmoid(a[..., 1]), _softplus(a[..., 2])


def aggregate(z, w_out, K_T):
    """App. C.4: the first K_T P columns of W_out applied to the concatenated z, times K_T^-1/2.
    z [B, K, P] (channels < K_T used); w_out [d, K, P]  ->  [B, d]."""
    return np.einsum("okp,bkp->bo", w_out[:, :K_T], z[:, :K_T]) / np.sqrt(K_T)


def decode_fused(state, u, w_in, beta, eps, w_ctl, b_ctl, rho, theta, c, w_out, K_T=None, zl=None):
    """One token through NL independent mixer layers, projections included.

    Returns (z [NL, B, K, P] (channels >= K_T zero), y [NL, B, d], new_state); channels >= K_T
    of the returned state keep their old values."""
    from . import decode_step   # the C oracle's mode recurrence (Eq. 5) and readout (Eq. 9, 24)
    NL, B, d = u.shape
    K, P = w_in.shape[1], w_in.shape[2]
    m = rho.shape[2]
    kt = K if K_T is None else int(K_T)
    v = np.zeros((NL, B, K, P))
    dl = np.zeros((NL, B, K, m))
    gw = np.zeros((NL, B, K, m))
    gr = np.zeros((NL, B, K, m))
    for l in range(NL):
        v[l, :, :kt] = channel_values(u[l], w_in[l], beta[l], eps, kt)
        gw[l, :, :kt], gr[l, :, :kt], dl[l, :, :kt] = controls(u[l], w_ctl[l], b_ctl[l], kt)
    z, st = decode_step(state, v, dl, gw, gr, rho, theta, c, K_T=kt, zl=zl)
    z[:, :, kt:] = 0.0
    y = np.stack([aggregate(z[l], w_out[l], kt) for l in range(NL)])
    return z, y, st
