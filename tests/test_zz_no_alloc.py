"""The allocation-free prefill entry point against the workspace one (needs an MI355X).

essh_mixer_prefill_noalloc keeps its look-back records in a static device array shared by
every call on the GPU.  Calls in a row, each smaller than the one before and then a large
one again, must give what essh_mixer_prefill gives with a workspace of its own: bit for bit
where the scan is deterministic (the three-launch segmented scan), and within the bf16
parity tolerance where the look-back may fold its predecessors in another order.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from selective_spectral_ssm_amd import inputs as I
from tests.gpu_util import TOL, block_err, device_inputs, to_dev, to_host_f64

pytestmark = pytest.mark.gpu

# (label, workload, shape overrides, K_T, with an entering state, comparison)
CASES = [
    ("three-launch 1 x 32768, K_T = 6", 4, dict(L=32768), 6, False, "exact"),
    ("look-back 2 x 2048, K_T = 24", 1, dict(B=2), 24, False, "tol"),
    ("three-launch 1 x 8192, K_T = 4, state_in", 4, dict(L=8192), 4, True, "exact"),
]


def log(msg: str):
    sys.__stderr__.write(f"[gpu-test] {msg}\n")
    sys.__stderr__.flush()


def _prepare(case):
    import torch
    from selective_spectral_ssm_amd import essh
    label, wi, over, K_T, with_state, kind = case
    w = I.workload(wi, **over)
    inp = I.make_prefill_inputs(w)
    d = device_inputs(inp)
    s_in = None
    if with_state:
        rng = np.random.default_rng(7)
        s_in = to_dev(rng.standard_normal((w.B, w.K, w.m, 2, w.P)).astype(np.float32))
    dims = essh.make_dims(w.B, w.L, w.K, w.m, w.P, K_T, w.Lc)
    need = essh.essh_prefill_workspace_bytes(dims)
    assert 0 < need <= essh.NOALLOC_SCRATCH_BYTES, (label, need)
    args = (d["v"], d["delta"], d["g_w"], d["g_r"], d["rho"], d["theta"], d["c"], None, s_in)
    return label, w, K_T, kind, dims, need, args


def _reference(prep):
    import torch
    from selective_spectral_ssm_amd import essh
    label, w, K_T, kind, dims, need, args = prep
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    y = torch.zeros_like(args[0])
    st = torch.zeros((w.B, w.K, w.m, 2, w.P), dtype=torch.float32, device="cuda")
    assert essh.essh_mixer_prefill(dims, *args, st, y, ws, need) == essh.ESSH_OK
    torch.cuda.synchronize()
    essh.check_workspace(ws)
    return y, st


def _noalloc(prep, err):
    import torch
    from selective_spectral_ssm_amd import essh
    label, w, K_T, kind, dims, need, args = prep
    y = torch.zeros_like(args[0])
    st = torch.zeros((w.B, w.K, w.m, 2, w.P), dtype=torch.float32, device="cuda")
    assert essh.essh_mixer_prefill_noalloc(dims, *args, st, y, scan_error=err) == essh.ESSH_OK
    return y, st


def _compare(prep, got, ref):
    import torch
    label, w, K_T, kind, dims, need, args = prep
    (y, st), (y_ref, st_ref) = got, ref
    if kind == "exact":
        diff = y.view(torch.int16) != y_ref.view(torch.int16)
        if diff.any():
            idx = diff.nonzero()
            log(f"{label}: {int(diff.sum())} y elements differ at positions {idx[:, 1].unique()[:16].tolist()}, "
                f"channels {idx[:, 2].unique().tolist()}; max |dy| "
                f"{float((y.float() - y_ref.float()).abs().max()):.3e}")
        assert not diff.any(), label
        assert torch.equal(st, st_ref), label
    else:
        ey = block_err(to_host_f64(y)[:, :, :K_T], to_host_f64(y_ref)[:, :, :K_T], chan_axis=2)
        es = block_err(to_host_f64(st)[:, :K_T], to_host_f64(st_ref)[:, :K_T], chan_axis=1)
        log(f"{label}: y err {ey:.2e}, state err {es:.2e} against the workspace call")
        assert ey <= TOL[w.io] and es <= TOL[w.io], label
        # channels past K_T untouched
        assert torch.count_nonzero(y[:, :, K_T:].float()) == 0 and torch.count_nonzero(st[:, K_T:]) == 0


def test_noalloc_matches_workspace_prefill_on_successive_calls():
    import torch
    preps = [_prepare(c) for c in CASES]
    refs = [_reference(p) for p in preps]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    # large, smaller, smaller, then the first again after the array held other dims
    for i in (0, 1, 2, 0):
        log(f"noalloc call: {preps[i][0]} (needs {preps[i][5]} bytes of scratch)")
        got = _noalloc(preps[i], err)
        torch.cuda.synchronize()
        _compare(preps[i], got, refs[i])
    assert int(err.item()) == 0
