"""The CPU oracle against what the paper and the mathematics fix (runs without a GPU).

Paper: "Elastic Selective Spectral Hybrids for Train-Once, Export-Many Budgeted
Inference" (ESSH).  See tests/oracle_pins.py for what each pin checks.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import reference
from tests.oracle_pins import ALL_PINS, _rand

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("name,pin,kw", ALL_PINS, ids=[p[0] for p in ALL_PINS])
def test_pin(name, pin, kw):
    err, tol = pin(oracle.prefill, **kw)
    assert err <= tol, f"{name}: error {err:.3e} > {tol:.1e}"


def test_resume_split_is_exact():
    """The state is the checkpoint: prefill(0:L1) -> state -> prefill(L1:L) equals prefill(0:L) exactly."""
    x = _rand(21, B=2, L=70, K=3, m=4, P=5)
    y, st = oracle.prefill(**x)
    L1 = 29
    first = {k: (v[:, :L1] if k in ("v", "delta", "g_w", "g_r") else v) for k, v in x.items()}
    rest = {k: (v[:, L1:] if k in ("v", "delta", "g_w", "g_r") else v) for k, v in x.items()}
    y1, s1 = oracle.prefill(**first)
    y2, s2 = oracle.prefill(**rest, state_in=s1)
    assert np.array_equal(np.concatenate([y1, y2], axis=1), y)
    assert np.array_equal(s2, st)


def test_truncation_is_exact_and_untouched():
    """Tier K_T reproduces the first K_T channels of the full mixer bit for bit (App. C.4, D.2),
    and channels k >= K_T of y and of the state are never written."""
    x = _rand(22, B=2, L=33, K=5, m=3, P=4)
    y_full, s_full = oracle.prefill(**x)
    for K_T in (1, 2, 4):
        sentinel = np.full(y_full.shape, 12345.0)
        y, st = oracle.prefill(**x, K_T=K_T, y_out=sentinel)
        assert np.array_equal(y[:, :, :K_T], y_full[:, :, :K_T])
        assert np.all(y[:, :, K_T:] == 12345.0)
        assert np.array_equal(st[:, :K_T], s_full[:, :K_T])
        assert np.all(st[:, K_T:] == 0.0)
    # NaN poisoning of discarded channels cannot reach retained ones
    xp = {k: np.array(v, copy=True) for k, v in x.items()}
    for key in ("v", "delta", "g_w", "g_r"):
        xp[key][:, :, 3:] = np.nan
    for key in ("rho", "theta", "c"):
        xp[key][3:] = np.nan
    y, st = oracle.prefill(**xp, K_T=3)
    assert np.array_equal(y[:, :, :3], y_full[:, :, :3])
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(st))


def test_per_mode_controls_broadcast():
    """Per-channel controls are the special case of per-mode controls with equal rows."""
    x = _rand(23, B=1, L=40, K=2, m=3, P=4)
    y, st = oracle.prefill(**x)
    xm = dict(x)
    for key in ("delta", "g_w", "g_r"):
        xm[key] = np.repeat(x[key][..., None], 3, axis=-1)
    y2, st2 = oracle.prefill(**xm)
    assert np.allclose(y2, y, rtol=0, atol=1e-14)
    assert np.allclose(st2, st, rtol=0, atol=1e-14)


def test_decode_step_extends_prefill():
    """A decode step after a prefill of L equals position L+1 of a prefill of L+1 (same recurrence)."""
    x = _rand(24, B=1, L=31, K=3, m=2, P=4)
    y_full, s_full = oracle.prefill(**x)
    L = 30
    head = {k: (v[:, :L] if k in ("v", "delta", "g_w", "g_r") else v) for k, v in x.items()}
    _, s = oracle.prefill(**head)
    yd, sd = oracle.decode_step(s[None], x["v"][None, :, L], x["delta"][None, :, L],
                                x["g_w"][None, :, L], x["g_r"][None, :, L],
                                x["rho"][None], x["theta"][None], x["c"][None])
    assert np.allclose(yd[0], y_full[:, L], rtol=0, atol=1e-13)
    assert np.allclose(sd[0], s_full, rtol=0, atol=1e-13)


def test_float32_build_tracks_float64():
    """The float32 build (CPU timing baseline only) computes the same thing to float32 accuracy."""
    x = _rand(25, B=2, L=128, K=3, m=4, P=8)
    y64, s64 = oracle.prefill(**x)
    y32, s32 = oracle.prefill_f32(**x)
    assert np.abs(y32 - y64).max() / np.abs(y64).max() < 1e-5
    assert np.abs(s32 - s64).max() / np.abs(s64).max() < 1e-5


def test_threads_parallel_identical():
    """OpenMP over independent (b, k) pairs gives identical results (channels are independent)."""
    x = _rand(26, B=3, L=50, K=4, m=2, P=3)
    y1, s1 = oracle.prefill(**x, nthreads=1)
    y4, s4 = oracle.prefill(**x, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(s1, s4)


def _read_table53():
    rows = []
    with open(os.path.join(GOLDEN, "table53_state_mb.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                tier, kt, mb = line.split()
                rows.append((tier, int(kt), float(mb)))
    return rows


def test_state_size_matches_table53():
    """Recurrent state per sequence: 2 K_T m P fp32 entries per spectral layer (Sec. 4.3),
    25 spectral layers, m=8, P=64 at the 1.5B scale -> the paper's Table 53 MB column."""
    from selective_spectral_ssm_amd.sizes import state_bytes
    for tier, kt, mb in _read_table53():
        got = state_bytes(n_layers=25, B=1, K=kt, m=8, P=64) / 1e6
        assert round(got, 2) == mb, (tier, got, mb)


def test_chunked_reference_matches_at_several_chunk_lengths():
    """Chunk boundaries anywhere: Lc in {1, 5, 64} (1 = every position is a chunk; 64 > L = one chunk)."""
    x = _rand(27, B=1, L=41, K=2, m=3, P=3)
    y, st = oracle.prefill(**x)
    for Lc in (1, 5, 64):
        yc, sc = reference.chunked(**x, Lc=Lc)
        assert np.abs(yc - y).max() <= 1e-12 * np.abs(y).max()
        assert np.abs(sc - st).max() <= 1e-12 * np.abs(st).max()


def test_decode_step_multilayer_tier_against_real_form():
    """oracle.decode_step over 3 layers with distinct mode tables, per-layer states and K_T < K,
    against the real 2xP rotation form of Eq. 5 (reference.real_form, a separate route) run one
    position per layer from that layer's state; channels k >= K_T keep their old state."""
    rng = np.random.default_rng(41)
    NL, B, K, m, P, K_T = 3, 2, 5, 3, 4, 3
    xs = [_rand(100 + l, B=B, L=1, K=K, m=m, P=P) for l in range(NL)]
    state = rng.normal(size=(NL, B, K, m, 2, P))
    stack = lambda key: np.stack([x[key][:, 0] if key in ("v", "delta", "g_w", "g_r") else x[key] for x in xs])
    y, st = oracle.decode_step(state, stack("v"), stack("delta"), stack("g_w"), stack("g_r"),
                               stack("rho"), stack("theta"), stack("c"), K_T=K_T)
    for l in range(NL):
        yr, sr = reference.real_form(**xs[l], K_T=K_T, state_in=state[l])
        assert np.abs(y[l][:, :K_T] - yr[:, 0, :K_T]).max() <= 1e-12 * np.abs(yr).max()
        assert np.abs(st[l][:, :K_T] - sr[:, :K_T]).max() <= 1e-12 * np.abs(sr[:, :K_T]).max()
        assert np.array_equal(st[l][:, K_T:], state[l][:, K_T:])
    # distinct layers really differ, so a layer-index slip cannot pass
    assert np.abs(y[0] - y[1]).max() > 1e-3


def test_decode_step_zero_lag_multilayer_against_jrec():
    """The zero-lag corrected decode step (Eq. 24) per layer against the App. C.3 J recurrence."""
    rng = np.random.default_rng(43)
    NL, B, K, m, P, K_T = 2, 1, 4, 2, 3, 4
    xs = [_rand(200 + l, B=B, L=1, K=K, m=m, P=P) for l in range(NL)]
    zl = rng.uniform(0.0, 1.0, size=(NL, K, m))
    state = rng.normal(size=(NL, B, K, m, 2, P))
    stack = lambda key: np.stack([x[key][:, 0] if key in ("v", "delta", "g_w", "g_r") else x[key] for x in xs])
    y, st = oracle.decode_step(state, stack("v"), stack("delta"), stack("g_w"), stack("g_r"),
                               stack("rho"), stack("theta"), stack("c"), K_T=K_T, zl=zl)
    for l in range(NL):
        # J(-1) = H(-1) - a b(-1); with one position, the state entering is H(-1) and b(-1)
        # is not part of this call, so start the J recurrence from H(-1) itself
        yr, sr = reference.zero_lag_jrec(**xs[l], zl=zl[l], K_T=K_T, state_in=state[l])
        assert np.abs(y[l] - yr[:, 0]).max() <= 1e-12 * np.abs(yr).max()
        assert np.abs(st[l] - sr).max() <= 1e-12 * np.abs(sr).max()
