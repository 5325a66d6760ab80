"""The fused decode step with projections against the oracle extension (needs an MI355X).

GPU: essh_decode_fused_step through the C ABI.  Oracle: oracle/fused.py in float64 on the same
bf16 weights and inputs (exact upcasts).  Everything after the bf16 inputs is fp32 on the GPU,
so besides the 2e-2 acceptance bound of bf16 inputs the errors are held to 1e-4 as a
regression bound (measured about 1e-6).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from selective_spectral_ssm_amd import inputs as I
from tests.gpu_util import TOL, block_err, to_dev, to_host_f64

pytestmark = pytest.mark.gpu

REGRESSION = 1e-4

# (name, NL, B, K, m, P, d_model, io, tiers)
CASES = [("small_bf16", 2, 2, 4, 4, 32, 128, "bf16", (4, 2)),
         ("width_not_k_times_p_f32", 1, 3, 3, 2, 16, 200, "f32", (3,)),
         ("m1_p64", 2, 1, 2, 1, 64, 64, "bf16", (2, 1)),
         ("m8_p128_width_1000", 1, 2, 3, 8, 128, 1000, "bf16", (3,)),
         # the decode workload's layer shape (K=32, m=8, P=128, d = K P = 4096), two layers
         ("decode_layer_shape", 2, 1, 32, 8, 128, 4096, "bf16", (32, 8)),
         # more than 256 channel workgroups (3 layers x 3 batch rows x 32 channels): the four-wave
         # launch shape of the per-channel projections; at K_T = 8 (72 workgroups) the eight-wave one
         ("many_channel_workgroups", 3, 3, 32, 8, 128, 4096, "bf16", (32, 8))]


def log(msg):
    sys.__stderr__.write(f"[gpu-test] {msg}\n")
    sys.__stderr__.flush()


def _err(got, ref):
    """max over (layer, batch row) of max|got - ref| / max|ref|"""
    g = got.reshape(got.shape[0] * got.shape[1], -1)
    r = ref.reshape(ref.shape[0] * ref.shape[1], -1)
    s = np.abs(r).max(axis=1)
    s = np.where(s > 0, s, 1.0)
    return float((np.abs(g - r).max(axis=1) / s).max())


@pytest.mark.parametrize("name,NL,B,K,m,P,D,io,tiers", CASES, ids=[c[0] for c in CASES])
def test_decode_fused_matches_oracle(name, NL, B, K, m, P, D, io, tiers):
    import torch
    from oracle import fused
    from selective_spectral_ssm_amd import essh
    x = I.make_fused_decode_inputs(NL, B, K, m, P, D, io)
    f64 = {k: I.as_f64(x[k], io if k == "u" else "bf16") for k in ("u", "w_in", "w_ctl", "w_out")}
    dev = {k: to_dev(x[k]) for k in ("u", "w_in", "w_ctl", "w_out", "beta", "b_ctl", "rho", "theta", "c", "zl")}
    eps = 1e-5
    for K_T in tiers:
        for zl in (None, x["zl"]):
            st = to_dev(x["state"].copy())
            z = torch.full((NL, B, K, P), 7.0, dtype=torch.float32, device="cuda")
            y = torch.empty((NL, B, D), dtype=torch.float32, device="cuda")
            dims = essh.make_dims(B, 1, K, m, P, K_T, 0, False, io)
            rc = essh.essh_decode_fused_step(NL, dims, D, dev["u"], dev["w_in"], dev["beta"], eps, dev["w_ctl"],
                                             dev["b_ctl"], dev["rho"], dev["theta"], dev["c"],
                                             None if zl is None else dev["zl"], dev["w_out"], st, z, y)
            assert rc == essh.ESSH_OK
            torch.cuda.synchronize()
            z_ref, y_ref, s_ref = fused.decode_fused(x["state"].astype(np.float64), f64["u"], f64["w_in"],
                                                     x["beta"].astype(np.float64), eps, f64["w_ctl"],
                                                     x["b_ctl"].astype(np.float64), x["rho"].astype(np.float64),
                                                     x["theta"].astype(np.float64), x["c"].astype(np.float64),
                                                     f64["w_out"], K_T=K_T,
                                                     zl=None if zl is None else zl.astype(np.float64))
            zg, sg, yg = to_host_f64(z), to_host_f64(st), to_host_f64(y)
            ez = max(block_err(zg[l, :, :K_T], z_ref[l, :, :K_T], chan_axis=1) for l in range(NL))
            es = max(block_err(sg[l, :, :K_T], s_ref[l, :, :K_T], chan_axis=1) for l in range(NL))
            ey = _err(yg, y_ref)
            log(f"{name} K_T={K_T} zero-lag={zl is not None}: z err {ez:.2e}, state err {es:.2e}, y err {ey:.2e}")
            assert max(ez, es, ey) <= TOL["bf16"]
            assert max(ez, es, ey) <= REGRESSION
            # channels past the tier: neither written nor updated
            assert torch.all(z[:, :, K_T:] == 7.0)
            assert np.array_equal(sg[:, :, K_T:], x["state"][:, :, K_T:].astype(np.float64))
