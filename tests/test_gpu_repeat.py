"""Repeatability of the three-launch prefill for few, long sequences (needs an MI355X).

The one-wave kernel stages each block of v in LDS by asynchronous global-to-LDS copies into a
ring of stages, stages y in place over it, and reads y back before the copies of a later block
overwrite the stage.  The copies must not overtake those reads: if they did, a few calls in a
hundred would store v rows (the segment's last row, which copies past its end repeat) as y.
Identical calls must therefore give identical y and state, bit for bit, every time.
"""
from __future__ import annotations

import sys

import pytest

from selective_spectral_ssm_amd import inputs as I
from tests.gpu_util import device_inputs

pytestmark = pytest.mark.gpu

# (workload overrides, K_T, calls): two-block segments at 32768 positions, and the 128K-token shape
CASES = [(dict(L=32768), 6, 500), (dict(), 24, 500)]


def log(msg: str):
    sys.__stderr__.write(f"[gpu-test] {msg}\n")
    sys.__stderr__.flush()


@pytest.mark.parametrize("over,K_T,calls", CASES, ids=["1x32768_kt6", "1x131072_kt24"])
def test_three_launch_prefill_is_repeatable(over, K_T, calls):
    import torch
    from selective_spectral_ssm_amd import essh
    w = I.workload(4, **over)
    d = device_inputs(I.make_prefill_inputs(w))
    dims = essh.make_dims(w.B, w.L, w.K, w.m, w.P, K_T, w.Lc)
    need = essh.essh_prefill_workspace_bytes(dims)
    args = (d["v"], d["delta"], d["g_w"], d["g_r"], d["rho"], d["theta"], d["c"], None, None)
    log(f"{w.name} L={w.L} K_T={K_T}: {calls} identical calls")
    y0 = s0 = None
    bad = []
    spacers = []
    for r in range(calls):
        # a fresh workspace every call, at an address moved by a spacer allocation
        spacers.append(torch.empty(((r * 7919) % 4093 + 1) * 1024, dtype=torch.uint8, device="cuda"))
        if len(spacers) > 4:
            spacers.pop(0)
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        y = torch.zeros_like(d["v"])
        st = torch.zeros((w.B, w.K, w.m, 2, w.P), dtype=torch.float32, device="cuda")
        assert essh.essh_mixer_prefill(dims, *args, st, y, ws, need) == essh.ESSH_OK
        torch.cuda.synchronize()
        essh.check_workspace(ws)
        yi = y.view(torch.int16)
        if y0 is None:
            y0, s0 = yi, st
            continue
        diff = yi != y0
        if diff.any() or not torch.equal(st, s0):
            idx = diff.nonzero()
            bad.append((r, int(diff.sum()), idx[:, 1].unique()[:8].tolist(), idx[:, 2].unique().tolist()))
    assert not bad, f"calls that differ from the first (call, elements, positions, channels): {bad[:5]}"
