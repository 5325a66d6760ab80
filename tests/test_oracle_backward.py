"""Pins of the backward oracle (oracle/backward.py), CPU only.

The gradients are checked against centred finite differences of the C oracle's forward pass in
float64 with step 1e-6, the check the ESSH paper reports for its own recurrence gradients
(App. "Numerical verification", Table 49: fp64, seed 2333, centred differences).  The forward
it differentiates is the independently pinned C oracle, so a mistake anywhere in the adjoint
(a dropped conjugate, a shifted decay, a missing term, a wrong sign) moves some gradient entry
away from the difference quotient.  Every entry of every input is perturbed.  Further pins:
the loss is linear in (v, state_in) jointly for fixed controls, so for those the difference
quotient is exact up to rounding; truncation to K_T gives zero gradients to discarded channels
and leaves the retained ones equal to those of the K_T-channel mixer.
"""
import numpy as np
import pytest

import oracle
from oracle.backward import prefill_backward

STEP = 1e-6
FD_TOL = 1e-7          # absolute; the paper's fp64 check reports 2.28e-9 at its shapes


def _case(seed=2333, B=2, L=9, K=3, m=2, P=3, per_mode=False, zl=False, state=True):
    rng = np.random.default_rng(seed)
    cs = (B, L, K, m) if per_mode else (B, L, K)
    x = dict(
        v=rng.normal(0, 1, (B, L, K, P)),
        delta=np.log1p(np.exp(rng.normal(0, 1, cs))),
        g_w=2.0 / (1.0 + np.exp(-rng.normal(0, 1, cs))),
        g_r=2.0 / (1.0 + np.exp(-rng.normal(0, 1, cs))),
        rho=rng.uniform(0.9, 0.999, (K, m)),
        theta=rng.uniform(0, np.pi, (K, m)),
        c=rng.normal(0, np.sqrt(1 / (2 * m)), (K, m, 2)),
    )
    if zl:
        x["zl"] = rng.uniform(0, 1, (K, m))
    if state:
        x["state_in"] = rng.normal(0, 1, (B, K, m, 2, P))
    dy = rng.normal(0, 1, (B, L, K, P))
    dso = rng.normal(0, 1, (B, K, m, 2, P))
    return x, dy, dso


def _loss(x, dy, dso, K_T):
    y, st = oracle.prefill(**x, K_T=K_T)
    return float(np.sum(y * dy) + np.sum(st * dso))


def _fd_grad(x, key, dy, dso, K_T, step=STEP):
    base = x[key]
    g = np.zeros_like(base)
    for idx in np.ndindex(base.shape):
        xp = dict(x)
        a = np.array(base, copy=True)
        a[idx] += step
        xp[key] = a
        lp = _loss(xp, dy, dso, K_T)
        a[idx] -= 2 * step
        lm = _loss(xp, dy, dso, K_T)
        g[idx] = (lp - lm) / (2 * step)
    return g


GRAD_OF = dict(v="dv", delta="ddelta", g_w="dg_w", g_r="dg_r", rho="drho", theta="dtheta", c="dc",
               state_in="dstate_in", zl="dzl")


@pytest.mark.parametrize("per_mode,zl", [(False, False), (False, True), (True, False), (True, True)],
                         ids=["channel", "channel_zl", "mode", "mode_zl"])
def test_gradients_match_centred_differences(per_mode, zl):
    x, dy, dso = _case(per_mode=per_mode, zl=zl)
    K_T = 2
    g = prefill_backward(**x, dy=dy, dstate_out=dso, K_T=K_T)
    worst = {}
    for key in x:
        fd = _fd_grad(x, key, dy, dso, K_T)
        err = float(np.max(np.abs(g[GRAD_OF[key]] - fd)))
        worst[key] = err
        assert err <= FD_TOL, f"d/d{key}: max abs error {err:.3e} against centred differences"
    # the check is not vacuous: every gradient has entries far above the tolerance
    for key in x:
        assert np.max(np.abs(g[GRAD_OF[key]])) > 1e-2, key


def test_forward_of_backward_is_the_oracle():
    """The forward states the backward pass builds are the C oracle's, to rounding."""
    for per_mode, zl in [(False, True), (True, True)]:
        x, dy, dso = _case(seed=5, per_mode=per_mode, zl=zl)
        g = prefill_backward(**x, dy=dy, dstate_out=dso, K_T=3)
        y, st = oracle.prefill(**x, K_T=3)
        assert np.max(np.abs(g["y"] - y)) < 1e-12
        assert np.max(np.abs(g["state_out"] - st)) < 1e-12


def test_linear_inputs_exact():
    """For fixed controls the loss is linear in (v, state_in): a difference quotient with a large
    step is then exact up to rounding, which pins dv and dstate_in at 1e-12 rather than 1e-7."""
    x, dy, dso = _case(seed=7, zl=True)
    g = prefill_backward(**x, dy=dy, dstate_out=dso, K_T=3)
    for key in ("v", "state_in"):
        fd = _fd_grad(x, key, dy, dso, 3, step=0.5)
        assert np.max(np.abs(g[GRAD_OF[key]] - fd)) < 1e-11, key


def test_no_state_arguments():
    """Without state_in the entering state is zero; without dstate_out the final state carries no
    gradient (the loss sees y only)."""
    x, dy, _ = _case(seed=9, state=False)
    g = prefill_backward(**x, dy=dy, K_T=3)
    zero = np.zeros_like(_case(seed=9)[2])
    for key in ("v", "delta", "theta"):
        fd = _fd_grad(x, key, dy, zero, 3)
        assert np.max(np.abs(g[GRAD_OF[key]] - fd)) <= FD_TOL, key


def test_truncation():
    """Channels k >= K_T get zero gradients (they are never computed); retained channels get the
    gradients of the K_T-channel mixer, bit for bit."""
    x, dy, dso = _case(seed=11, K=4, zl=True)
    K_T = 2
    g = prefill_backward(**x, dy=dy, dstate_out=dso, K_T=K_T)
    xs = {k: (a[:, :, :K_T] if k in ("v", "delta", "g_w", "g_r") else
              a[:, :K_T] if k == "state_in" else a[:K_T]) for k, a in x.items()}
    gs = prefill_backward(**xs, dy=dy[:, :, :K_T], dstate_out=dso[:, :K_T])
    for key, name in GRAD_OF.items():
        full = g[name]
        ax = 2 if key in ("v", "delta", "g_w", "g_r") else 1 if key == "state_in" else 0
        keep = np.take(full, range(K_T), axis=ax)
        drop = np.take(full, range(K_T, 4), axis=ax)
        assert np.array_equal(keep, gs[name]), key
        assert np.all(drop == 0.0), key


def test_empty_sequence():
    """L = 0: no positions, so dstate_in is dstate_out and every other gradient is zero."""
    x, dy, dso = _case(seed=3, L=0, zl=True)
    g = prefill_backward(**x, dy=dy, dstate_out=dso)
    assert np.array_equal(g["dstate_in"], dso)
    for name in ("dv", "ddelta", "dg_w", "dg_r", "drho", "dtheta", "dc", "dzl"):
        assert np.all(g[name] == 0.0), name


MUTANTS = [
    ("adjoint decay not conjugated", "ab = np.conj(lam(t))[..., None] * ab", "ab = lam(t)[..., None] * ab"),
    ("readout coefficient not conjugated", "* np.conj(cc)[None, :, :, None]", "* cc[None, :, :, None]"),
    ("pole-magnitude chain rule inverted", "axis=(0, 3)) / rr", "axis=(0, 3)) * rr"),
    ("adjoint not conjugated in the transition term", "inner = np.conj(ab) *", "inner = ab *"),
    ("transition term on h(t) instead of h(t-1)", "hprev = h[t - 1] if t > 0 else h_init",
     "hprev = h[t]"),
    ("zero-lag gradient sign", "dzl[sl] -= ", "dzl[sl] += "),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistakes_are_caught(name, old, new):
    """Each plausible mistake, planted in a copy of the backward oracle, fails the
    centred-difference pin on at least one input."""
    import inspect
    import types
    from oracle import backward
    src = inspect.getsource(backward)
    assert src.count(old) == 1, name
    mod = types.ModuleType("backward_mutant")
    exec(compile(src.replace(old, new), "backward_mutant", "exec"), mod.__dict__)
    x, dy, dso = _case(seed=17, zl=True, L=5)
    g = mod.prefill_backward(**x, dy=dy, dstate_out=dso, K_T=2)
    worst = max(float(np.max(np.abs(g[GRAD_OF[key]] - _fd_grad(x, key, dy, dso, 2)))) for key in x)
    assert worst > 1e3 * FD_TOL, f"{name}: survived the pin (max error {worst:.2e})"
