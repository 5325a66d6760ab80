"""Pins of the fused-decode oracle extension (oracle/fused.py), CPU only.

Each part is checked against something other than itself: brute-force loops over the
definition, closed forms the pages state, the pages' own initial values (tests/golden/), the
reduction to the C oracle's decode step with the controls given directly, and the truncation
property of App. C.4.  Planted mistakes (a gate without its factor 2, a blend statistic over all
channels, an exponential clock, a missing K_T^-1/2) are each caught by one of the pins.
"""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import fused

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "c2_initial_clock.txt")


def _case(NL=2, B=2, K=3, m=2, P=4, d=12, seed=0):
    rng = np.random.default_rng(seed)
    u = rng.normal(0, 1, (NL, B, d))
    w_in = rng.normal(0, 0.3, (NL, K, P, d))
    beta = rng.uniform(-0.5, 1.5, (NL, K))
    w_ctl = rng.normal(0, 0.3, (NL, K, m, 3, d))
    b_ctl = rng.normal(0, 1.0, (NL, K, m, 3))
    rho = rng.uniform(0.9, 0.999, (NL, K, m))
    theta = rng.uniform(0, np.pi, (NL, K, m))
    c = rng.normal(0, np.sqrt(1 / (2 * m)), (NL, K, m, 2))
    zl = rng.uniform(0, 1, (NL, K, m))
    w_out = rng.normal(0, 0.3, (NL, d, K, P))
    state = rng.normal(0, 1, (NL, B, K, m, 2, P))
    return dict(u=u, w_in=w_in, beta=beta, w_ctl=w_ctl, b_ctl=b_ctl, rho=rho, theta=theta, c=c, zl=zl,
                w_out=w_out, state=state)


# ---- channel values (Eq. 23) -----------------------------------------------------------------

def check_blend(channel_values) -> bool:
    """Brute-force Eq. 23 per element, its beta = 0 and beta = 1 closed forms, channel locality."""
    cs = _case()
    u, w_in = cs["u"][0], cs["w_in"][0]
    B, K, P, d = u.shape[0], w_in.shape[0], w_in.shape[1], w_in.shape[2]
    eps = 1e-3
    ok = True
    for beta_val in (0.0, 1.0, 0.3):
        beta = np.full(K, beta_val)
        v = channel_values(u, w_in, beta, eps, K)
        for b in range(B):
            for k in range(K):
                v0 = [sum(w_in[k, p, e] * u[b, e] for e in range(d)) for p in range(P)]
                ms = sum(x * x for x in v0) / P
                for p in range(P):
                    want = (1 - beta_val) * v0[p] + beta_val * v0[p] / math.sqrt(ms + eps)
                    ok &= abs(v[b, k, p] - want) <= 1e-12 * (1 + abs(want))
                if beta_val == 1.0:   # RMS of the normalized value is sqrt(ms / (ms + eps))
                    ok &= abs(np.mean(v[b, k] ** 2) - ms / (ms + eps)) <= 1e-12
    # another channel's rows do not change channel 0's value
    w2 = w_in.copy()
    w2[1:] *= -3.0
    beta = np.full(K, 0.7)
    ok &= bool(np.array_equal(channel_values(u, w_in, beta, eps, K)[:, 0], channel_values(u, w2, beta, eps, K)[:, 0]))
    return bool(ok)


def test_blend():
    assert check_blend(fused.channel_values)


# ---- gates and clock (App. C.2) --------------------------------------------------------------

def check_controls(controls) -> bool:
    stated = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, val, digits = line.split()
        stated[name] = (float(val), int(digits))
    K, m, d = 3, 2, 8
    u = np.random.default_rng(1).normal(0, 1, (2, d))
    w = np.zeros((K, m, 3, d))
    b = np.zeros((K, m, 3))
    b[..., 2] = -3.0
    gw, gr, dl = controls(u, w, b, K)
    ok = True
    ok &= bool(np.all(gw == stated["gate_value"][0]) and np.all(gr == stated["gate_value"][0]))
    # each stated value rounded to the decimals it is stated with
    val, dec = stated["clock_increment"]
    ok &= abs(dl[0, 0, 0] - val) <= 0.5 * 10.0 ** (-dec)
    val, dec = stated["efolding_positions"]
    ok &= abs(1.0 / dl[0, 0, 0] - val) <= 0.5 * 10.0 ** (-dec)
    # per element against the math library, with large arguments
    rng = np.random.default_rng(2)
    w = rng.normal(0, 1, (K, m, 3, d))
    b = rng.normal(0, 1, (K, m, 3))
    b[0, 0, 2] = 800.0
    b[0, 1, 2] = -800.0
    gw, gr, dl = controls(u, w, b, K)
    for bb in range(u.shape[0]):
        for k in range(K):
            for j in range(m):
                a = [sum(w[k, j, s, e] * u[bb, e] for e in range(d)) + b[k, j, s] for s in range(3)]
                ok &= abs(gw[bb, k, j] - 2 / (1 + math.exp(-a[0]))) <= 1e-12
                ok &= abs(gr[bb, k, j] - 2 / (1 + math.exp(-a[1]))) <= 1e-12
                sp = a[2] if a[2] > 30 else math.log1p(math.exp(a[2]))
                ok &= abs(dl[bb, k, j] - sp) <= 1e-12 * (1 + abs(sp))
    return bool(ok)


def test_controls():
    assert check_controls(fused.controls)


# ---- aggregation (App. C.4) ------------------------------------------------------------------

def check_aggregate(aggregate) -> bool:
    rng = np.random.default_rng(3)
    B, K, P, d = 2, 4, 3, 5
    z = rng.normal(0, 1, (B, K, P))
    w_out = rng.normal(0, 1, (d, K, P))
    ok = True
    for kt in (1, 3, 4):
        y = aggregate(z, w_out, kt)
        for b in range(B):
            for o in range(d):
                s = sum(w_out[o, k, p] * z[b, k, p] for k in range(kt) for p in range(P))
                ok &= abs(y[b, o] - s / math.sqrt(kt)) <= 1e-12 * (1 + abs(s))
    return bool(ok)


def test_aggregate():
    assert check_aggregate(fused.aggregate)


# ---- the whole step ----------------------------------------------------------------------------

def test_fused_reduces_to_decode_step_with_given_controls():
    """Selection rows for W_in (u holds the channel values), beta = 0, zero control weights and
    biases that produce given gates and clock: the step equals the C oracle's decode step run on
    those values and controls, and y is W_out z scaled by K_T^-1/2."""
    NL, B, K, m, P = 2, 2, 3, 2, 4
    d = K * P
    cs = _case(NL, B, K, m, P, d, seed=4)
    rng = np.random.default_rng(5)
    vals = rng.normal(0, 1, (NL, B, K, P))
    gw = rng.uniform(0.1, 1.9, (NL, B, K, m))
    gr = rng.uniform(0.1, 1.9, (NL, B, K, m))
    dl = rng.uniform(0.01, 2.0, (NL, B, K, m))
    # one batch row per call: the control biases are per channel and mode, not per batch row
    for b in range(B):
        u = vals[:, b].reshape(NL, 1, d)
        w_in = np.zeros((NL, K, P, d))
        for k in range(K):
            for p in range(P):
                w_in[:, k, p, k * P + p] = 1.0
        w_ctl = np.zeros((NL, K, m, 3, d))
        b_ctl = np.stack([np.log((gw[:, b] / 2) / (1 - gw[:, b] / 2)), np.log((gr[:, b] / 2) / (1 - gr[:, b] / 2)),
                          np.log(np.expm1(dl[:, b]))], axis=-1)
        st = cs["state"][:, b:b + 1]
        for kt in (K, 2):
            z, y, st2 = fused.decode_fused(st, u, w_in, np.zeros((NL, K)), 1e-5, w_ctl, b_ctl, cs["rho"], cs["theta"],
                                           cs["c"], cs["w_out"], K_T=kt, zl=cs["zl"])
            z_ref, st_ref = oracle.decode_step(st, vals[:, b:b + 1], dl[:, b:b + 1], gw[:, b:b + 1], gr[:, b:b + 1],
                                               cs["rho"], cs["theta"], cs["c"], K_T=kt, zl=cs["zl"])
            assert np.allclose(z[:, :, :kt], z_ref[:, :, :kt], rtol=1e-11, atol=1e-12)
            assert np.allclose(st2, st_ref, rtol=1e-11, atol=1e-12)
            for l in range(NL):
                for o in range(d):
                    s = sum(cs["w_out"][l, o, k, p] * z_ref[l, 0, k, p] for k in range(kt) for p in range(P))
                    assert abs(y[l, 0, o] - s / math.sqrt(kt)) <= 1e-10 * (1 + abs(s))


def test_fused_truncation_keeps_retained_channels():
    """App. C.4: at tier K_T the retained channels compute exactly what they compute at full
    width, and the output is their share of the full output rescaled."""
    cs = _case(NL=2, B=2, K=4, m=2, P=3, d=10, seed=6)
    args = (cs["state"], cs["u"], cs["w_in"], cs["beta"], 1e-3, cs["w_ctl"], cs["b_ctl"], cs["rho"], cs["theta"],
            cs["c"], cs["w_out"])
    z4, y4, s4 = fused.decode_fused(*args, K_T=4, zl=cs["zl"])
    z2, y2, s2 = fused.decode_fused(*args, K_T=2, zl=cs["zl"])
    assert np.array_equal(z2[:, :, :2], z4[:, :, :2])
    assert np.array_equal(s2[:, :, :2], s4[:, :, :2])
    assert np.array_equal(s2[:, :, 2:], cs["state"][:, :, 2:])
    assert np.all(z2[:, :, 2:] == 0)
    part = np.einsum("lokp,lbkp->lbo", cs["w_out"][:, :, :2], z4[:, :, :2])
    assert np.allclose(y2 * np.sqrt(2), part, rtol=1e-12, atol=1e-12)


# ---- planted mistakes -----------------------------------------------------------------------

def test_pins_catch_planted_mistakes():
    def blend_global(u, w_in, beta, eps, K_T):       # statistic over all retained channels
        v0 = np.einsum("kpd,bd->bkp", w_in[:K_T], u)
        ms = np.mean(v0 * v0, axis=(1, 2), keepdims=True)
        bt = beta[:K_T][None, :, None]
        return (1 - bt) * v0 + bt * v0 / np.sqrt(ms + eps)

    def blend_swapped(u, w_in, beta, eps, K_T):      # beta on the wrong term
        v0 = np.einsum("kpd,bd->bkp", w_in[:K_T], u)
        ms = np.mean(v0 * v0, axis=-1, keepdims=True)
        bt = beta[:K_T][None, :, None]
        return bt * v0 + (1 - bt) * v0 / np.sqrt(ms + eps)

    def controls_sigmoid(u, w_ctl, b_ctl, K_T):     # gates without the factor 2
        gw, gr, dl = fused.controls(u, w_ctl, b_ctl, K_T)
        return gw / 2, gr / 2, dl

    def controls_exp_clock(u, w_ctl, b_ctl, K_T):   # clock e^x instead of softplus
        a = np.einsum("kmsd,bd->bkms", w_ctl[:K_T], u) + b_ctl[:K_T][None]
        gw, gr, _ = fused.controls(u, w_ctl, b_ctl, K_T)
        return gw, gr, np.exp(np.minimum(a[..., 2], 50))

    def controls_swapped(u, w_ctl, b_ctl, K_T):     # write and read rows exchanged
        gw, gr, dl = fused.controls(u, w_ctl, b_ctl, K_T)
        return gr, gw, dl

    def aggregate_unscaled(z, w_out, K_T):
        return np.einsum("okp,bkp->bo", w_out[:, :K_T], z[:, :K_T])

    def aggregate_full_width_scale(z, w_out, K_T):
        return np.einsum("okp,bkp->bo", w_out[:, :K_T], z[:, :K_T]) / np.sqrt(w_out.shape[1])

    assert not check_blend(blend_global)
    assert not check_blend(blend_swapped)
    assert not check_controls(controls_sigmoid)
    assert not check_controls(controls_exp_clock)
    assert not check_controls(controls_swapped)
    assert not check_aggregate(aggregate_unscaled)
    assert not check_aggregate(aggregate_full_width_scale)
