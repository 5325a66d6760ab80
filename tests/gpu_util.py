"""Helpers shared by the GPU tests: device transfer of seeded inputs and error metrics."""
from __future__ import annotations

import numpy as np

from selective_spectral_ssm_amd.inputs import as_f64, bf16_bits_to_f32

# Tolerances stated for this method: fp32 inputs 1e-4, bf16 inputs with fp32 state 2e-2,
# both as a normalised maximum error (see block_err).
TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_dev(x: np.ndarray, device="cuda"):
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def to_host_f64(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        bits = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
        return bf16_bits_to_f32(bits).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def device_inputs(inp: dict, device="cuda") -> dict:
    return {k: to_dev(inp[k], device) for k in ("v", "delta", "g_w", "g_r", "rho", "theta", "c")}


def oracle_inputs(inp: dict) -> dict:
    """Exact float64 upcast of what the GPU reads (bf16 values already rounded)."""
    io = inp["io"]
    return dict(v=as_f64(inp["v"], io), delta=inp["delta"].astype(np.float64),
                g_w=as_f64(inp["g_w"], io), g_r=as_f64(inp["g_r"], io),
                rho=inp["rho"].astype(np.float64), theta=inp["theta"].astype(np.float64),
                c=inp["c"].astype(np.float64))


def block_err(got: np.ndarray, ref: np.ndarray, chan_axis: int, B_axis: int = 0) -> float:
    """Normalised max error: max over (b, k) of max|got - ref| / max|ref| within that channel block.

    Elementwise relative error is undefined at zero crossings; normalising each
    (batch row, channel) block by its own largest reference magnitude keeps a
    channel with small outputs from hiding behind a large one.
    """
    got = np.moveaxis(got, (B_axis, chan_axis), (0, 1))
    ref = np.moveaxis(ref, (B_axis, chan_axis), (0, 1))
    Bn, Kn = ref.shape[:2]
    d = np.abs(got - ref).reshape(Bn, Kn, -1).max(axis=2)
    s = np.abs(ref).reshape(Bn, Kn, -1).max(axis=2)
    s = np.where(s > 0, s, 1.0)
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float((d / s).max())
