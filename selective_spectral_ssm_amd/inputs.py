"""Seeded synthetic inputs for the selective spectral mixer core.

This module only draws numbers.  It holds none of the mixer's arithmetic: the
clock and gate draws are handed over already post-activation (the kernels and
the oracle never apply softplus or sigmoid themselves), and bf16 values are
produced by IEEE round-to-nearest-even from float32 so that the oracle can
consume the exact upcast of what the GPU reads.

Both the HIP path (through the Python binding) and the CPU oracle take their
inputs from here; neither side imports the other.

Workload shapes follow the five workloads of the selective spectral mixer
study (tiny fp32 mixer, 370M-class and 1.5B-class prefill layers, 24-layer
batch-one decode, 128K-token DNA-like prefill).  Distributions:
  v ~ N(0,1); delta = softplus(N(0,1)); g_w, g_r = sigmoid(N(0,1));
  rho ~ U(0.90, 0.999) (U(0.95, 0.9999) for the 1.5B-class shapes);
  theta ~ U(0, pi); c = c_re + i c_im with c_re, c_im ~ N(0, 1/(2m)) i.i.d.
The seed is 2333 + workload index (2333 is the seed of the paper's own
numerical verification table).  Draw order is fixed: rho, theta, c_re, c_im,
then the per-token arrays.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SEED_BASE = 2333


# ----------------------------------------------------------------------------
# bf16 helpers (bit patterns held in uint16 arrays; numpy has no bf16 dtype)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


# ----------------------------------------------------------------------------
# Workload descriptions
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    B: int
    L: int
    K: int
    m: int
    P: int
    Lc: int
    io: str                      # "f32" or "bf16" (dtype of v, g_w, g_r and y)
    rho_lo: float
    rho_hi: float
    tiers: tuple
    layers: int = 1              # decode workload: number of independent mixer layers
    steps: int = 0               # decode workload: tokens decoded after the context
    dna: bool = False            # long-sequence workload: v from 4-symbol tokens

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index


WORKLOADS = {
    0: Workload(0, "tiny_f32", B=1, L=256, K=8, m=4, P=16, Lc=64, io="f32",
                rho_lo=0.90, rho_hi=0.999, tiers=(8,)),
    1: Workload(1, "mixer370m_prefill", B=8, L=2048, K=24, m=4, P=64, Lc=64, io="bf16",
                rho_lo=0.90, rho_hi=0.999, tiers=(6, 12, 18, 24)),
    2: Workload(2, "mixer1p5b_prefill", B=16, L=2048, K=32, m=8, P=128, Lc=64, io="bf16",
                rho_lo=0.95, rho_hi=0.9999, tiers=(8, 16, 24, 32)),
    3: Workload(3, "mixer1p5b_decode", B=1, L=2048, K=32, m=8, P=128, Lc=64, io="bf16",
                rho_lo=0.95, rho_hi=0.9999, tiers=(8, 16, 24, 32), layers=24, steps=1024),
    4: Workload(4, "dna128k_prefill", B=1, L=131072, K=24, m=4, P=64, Lc=128, io="bf16",
                rho_lo=0.90, rho_hi=0.999, tiers=(6, 12, 18, 24), dna=True),
}


def workload(index: int, **overrides) -> Workload:
    """Return workload ``index``, optionally with some fields replaced (reduced shapes)."""
    w = WORKLOADS[index]
    return dataclasses.replace(w, **overrides) if overrides else w


# ----------------------------------------------------------------------------
# Draws
# ----------------------------------------------------------------------------

def draw_params(rng: np.random.Generator, K: int, m: int, rho_lo: float, rho_hi: float):
    """Mode tables: rho [K,m], theta [K,m], c [K,m,2] (re, im), all float32."""
    rho = rng.uniform(rho_lo, rho_hi, size=(K, m))
    theta = rng.uniform(0.0, np.pi, size=(K, m))
    s = np.sqrt(1.0 / (2.0 * m))
    c_re = rng.normal(0.0, s, size=(K, m))
    c_im = rng.normal(0.0, s, size=(K, m))
    c = np.stack([c_re, c_im], axis=-1)
    return (rho.astype(np.float32), theta.astype(np.float32), c.astype(np.float32))


def _io_array(x64: np.ndarray, io: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return f32_to_bf16_bits(x32) if io == "bf16" else x32


def draw_tokens(rng: np.random.Generator, B: int, L: int, K: int, P: int, io: str,
                per_mode_m: Optional[int] = None, dna: bool = False):
    """Per-token arrays: v [B,L,K,P], delta, g_w, g_r ([B,L,K] or [B,L,K,m])."""
    if dna:
        sym = rng.integers(0, 4, size=(B, L))
        E = rng.normal(0.0, 1.0, size=(4, K, P))
        v = _io_array(E, io)[sym]          # gather of already-rounded rows
    else:
        v = _io_array(rng.normal(0.0, 1.0, size=(B, L, K, P)), io)
    cshape = (B, L, K) if per_mode_m is None else (B, L, K, per_mode_m)
    delta = _softplus(rng.normal(0.0, 1.0, size=cshape)).astype(np.float32)
    g_w = _io_array(_sigmoid(rng.normal(0.0, 1.0, size=cshape)), io)
    g_r = _io_array(_sigmoid(rng.normal(0.0, 1.0, size=cshape)), io)
    return v, delta, g_w, g_r


def make_prefill_inputs(w: Workload, per_mode: bool = False, seed: Optional[int] = None) -> dict:
    """All inputs of one prefill call, drawn for the full channel count K.

    A tier K_T reads the first K_T channels of these arrays.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    rho, theta, c = draw_params(rng, w.K, w.m, w.rho_lo, w.rho_hi)
    v, delta, g_w, g_r = draw_tokens(rng, w.B, w.L, w.K, w.P, w.io,
                                     per_mode_m=w.m if per_mode else None, dna=w.dna)
    return dict(v=v, delta=delta, g_w=g_w, g_r=g_r, rho=rho, theta=theta, c=c,
                io=w.io, per_mode=per_mode)


def make_backward_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """Inputs of one backward call: the prefill inputs of ``w`` (per-channel controls), then
    dy ~ N(0,1) [B,L,K,P] in the io dtype, state_in and dstate_out ~ N(0,1) [B,K,m,2,P] fp32 and
    zero-lag coefficients zl ~ U(0,1) [K,m] fp32, drawn in that order."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    rho, theta, c = draw_params(rng, w.K, w.m, w.rho_lo, w.rho_hi)
    v, delta, g_w, g_r = draw_tokens(rng, w.B, w.L, w.K, w.P, w.io, dna=w.dna)
    dy = _io_array(rng.normal(0.0, 1.0, size=(w.B, w.L, w.K, w.P)), w.io)
    state_in = rng.normal(0.0, 1.0, size=(w.B, w.K, w.m, 2, w.P)).astype(np.float32)
    dstate_out = rng.normal(0.0, 1.0, size=(w.B, w.K, w.m, 2, w.P)).astype(np.float32)
    zl = rng.uniform(0.0, 1.0, size=(w.K, w.m)).astype(np.float32)
    return dict(v=v, delta=delta, g_w=g_w, g_r=g_r, rho=rho, theta=theta, c=c, dy=dy, state_in=state_in,
                dstate_out=dstate_out, zl=zl, io=w.io, per_mode=False)


def make_decode_inputs(w: Workload, n_steps: Optional[int] = None, context: Optional[int] = None,
                       seed: Optional[int] = None) -> dict:
    """Decode workload: per-layer params, a context to pre-fill the state, per-step tokens.

    Returns params with a leading layer axis (rho [NL,K,m] ...), context arrays
    [NL,B,Lctx,K,...] and step arrays [S,NL,B,K,...].
    """
    n_steps = w.steps if n_steps is None else n_steps
    context = w.L if context is None else context
    rng = np.random.default_rng(w.seed if seed is None else seed)
    NL = w.layers
    rho = np.empty((NL, w.K, w.m), np.float32)
    theta = np.empty_like(rho)
    c = np.empty((NL, w.K, w.m, 2), np.float32)
    for l in range(NL):
        rho[l], theta[l], c[l] = draw_params(rng, w.K, w.m, w.rho_lo, w.rho_hi)
    ctx = [draw_tokens(rng, w.B, context, w.K, w.P, w.io) for _ in range(NL)]
    cv, cd, cgw, cgr = (np.stack([x[i] for x in ctx]) for i in range(4))
    sv, sd, sgw, sgr = draw_tokens(rng, n_steps * NL, w.B, w.K, w.P, w.io)
    # draw_tokens returns [n_steps*NL, B, K, ...] as its (B, L) axes; regroup.
    sv = sv.reshape(n_steps, NL, w.B, w.K, w.P)
    sd = sd.reshape(n_steps, NL, w.B, w.K)
    sgw = sgw.reshape(n_steps, NL, w.B, w.K)
    sgr = sgr.reshape(n_steps, NL, w.B, w.K)
    return dict(rho=rho, theta=theta, c=c,
                ctx_v=cv, ctx_delta=cd, ctx_g_w=cgw, ctx_g_r=cgr,
                step_v=sv, step_delta=sd, step_g_w=sgw, step_g_r=sgr, io=w.io)


def make_fused_decode_inputs(NL: int, B: int, K: int, m: int, P: int, d_model: int, io: str = "bf16",
                             seed: int = SEED_BASE + 3, rho_lo: float = 0.95, rho_hi: float = 0.9999) -> dict:
    """Synthetic inputs of the fused decode step with projections (random-init weights of the
    layout the library takes, drawn as the decode workload draws its mode tables).

    u [NL,B,d] (io); w_in [NL,K,P,d], w_ctl [NL,K,m,3,d], w_out [NL,d,K,P] as bf16 bits, entries
    N(0, 1/fan_in); beta [NL,K] ~ U(-0.5, 1.5); b_ctl [NL,K,m,3]: gate biases N(0,1), clock
    biases N(-2, 1); rho, theta, c as the decode workload; zl [NL,K,m] ~ U(0,1);
    state [NL,B,K,m,2,P] ~ N(0,1) (fp32)."""
    rng = np.random.default_rng(seed)
    rho = np.empty((NL, K, m), np.float32)
    theta = np.empty_like(rho)
    c = np.empty((NL, K, m, 2), np.float32)
    for l in range(NL):
        rho[l], theta[l], c[l] = draw_params(rng, K, m, rho_lo, rho_hi)
    u = _io_array(rng.normal(0.0, 1.0, size=(NL, B, d_model)), io)
    w_in = f32_to_bf16_bits(rng.normal(0.0, 1.0 / np.sqrt(d_model), size=(NL, K, P, d_model)).astype(np.float32))
    w_ctl = f32_to_bf16_bits(rng.normal(0.0, 1.0 / np.sqrt(d_model), size=(NL, K, m, 3, d_model)).astype(np.float32))
    w_out = f32_to_bf16_bits(rng.normal(0.0, 1.0 / np.sqrt(K * P), size=(NL, d_model, K, P)).astype(np.float32))
    beta = rng.uniform(-0.5, 1.5, size=(NL, K)).astype(np.float32)
    b_ctl = rng.normal(0.0, 1.0, size=(NL, K, m, 3))
    b_ctl[..., 2] -= 2.0
    zl = rng.uniform(0.0, 1.0, size=(NL, K, m)).astype(np.float32)
    state = rng.normal(0.0, 1.0, size=(NL, B, K, m, 2, P)).astype(np.float32)
    return dict(u=u, w_in=w_in, w_ctl=w_ctl, w_out=w_out, beta=beta, b_ctl=b_ctl.astype(np.float32), rho=rho,
                theta=theta, c=c, zl=zl, state=state, io=io, d_model=d_model)


def as_f64(x: np.ndarray, io: str) -> np.ndarray:
    """Exact float64 view of an io array (bf16 bits or float32)."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)
