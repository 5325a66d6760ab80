"""GPU backward pass against the backward oracle, element by element, through the C ABI.

The oracle (oracle/backward.py) is float64 and pinned on the CPU by centred finite differences
of the forward oracle.  Both sides get the same seeded inputs (bf16 values already rounded).
Errors are per-(batch row, channel) normalised maxima (tests/gpu_util.py).  The mode-table
gradients are sums over every batch row and position, and one channel's sum can cancel to near
zero (with m = 1 a channel's block is that single sum), so their error is normalised by the
largest entry over all retained channels.  Bars: 1e-4 for fp32 io; 2e-2 for bf16 io (dv is
written in bf16; the other gradients are fp32 and held to 1e-4 as well).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle.backward import prefill_backward as oracle_backward
from selective_spectral_ssm_amd import inputs as I
from tests.gpu_util import TOL, block_err, to_dev, to_host_f64

pytestmark = pytest.mark.gpu

SENTINEL = 7.0
F32_GRAD_TOL = 1e-4


def log(msg: str):
    sys.__stderr__.write(f"[gpu-test] {msg}\n")
    sys.__stderr__.flush()


def run_gpu_backward(inp, K_T, use_state=True, use_zl=True):
    import torch
    from selective_spectral_ssm_amd import essh
    d = {k: to_dev(inp[k]) for k in ("v", "delta", "g_w", "g_r", "rho", "theta", "c", "dy")}
    s_in = to_dev(inp["state_in"]) if use_state else None
    dso = to_dev(inp["dstate_out"]) if use_state else None
    zl = to_dev(inp["zl"]) if use_zl else None
    B, L, K, P = inp["v"].shape
    m = inp["rho"].shape[1]
    dims = essh.make_dims(B, L, K, m, P, K_T, 0, False, inp["io"])
    f32 = dict(dtype=torch.float32, device="cuda")
    g = dict(dv=torch.full_like(d["v"], SENTINEL), ddelta=torch.full((B, L, K), SENTINEL, **f32),
             dg_w=torch.full((B, L, K), SENTINEL, **f32), dg_r=torch.full((B, L, K), SENTINEL, **f32),
             drho=torch.full((K, m), SENTINEL, **f32), dtheta=torch.full((K, m), SENTINEL, **f32),
             dc=torch.full((K, m, 2), SENTINEL, **f32), dzl=torch.full((K, m), SENTINEL, **f32),
             dstate_in=torch.full((B, K, m, 2, P), SENTINEL, **f32))
    ws_bytes = essh.essh_prefill_backward_workspace_bytes(dims)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    st = essh.essh_mixer_prefill_backward(dims, d["v"], d["delta"], d["g_w"], d["g_r"], d["rho"], d["theta"],
                                          d["c"], zl, s_in, d["dy"], dso, g["dv"], g["ddelta"], g["dg_w"],
                                          g["dg_r"], g["drho"], g["dtheta"], g["dc"], g["dzl"], g["dstate_in"],
                                          ws, ws_bytes)
    assert st == essh.ESSH_OK, essh.status_string(st)
    torch.cuda.synchronize()
    return {k: to_host_f64(t) for k, t in g.items()}


def oracle_grads(inp, K_T, use_state=True, use_zl=True):
    io = inp["io"]
    return oracle_backward(
        v=I.as_f64(inp["v"], io), delta=inp["delta"].astype(np.float64), g_w=I.as_f64(inp["g_w"], io),
        g_r=I.as_f64(inp["g_r"], io), rho=inp["rho"].astype(np.float64), theta=inp["theta"].astype(np.float64),
        c=inp["c"].astype(np.float64), dy=I.as_f64(inp["dy"], io), K_T=K_T,
        state_in=inp["state_in"].astype(np.float64) if use_state else None,
        dstate_out=inp["dstate_out"].astype(np.float64) if use_state else None,
        zl=inp["zl"].astype(np.float64) if use_zl else None)


CTRL_AXES = {"dv": 2, "ddelta": 2, "dg_w": 2, "dg_r": 2, "dstate_in": 1}
TABLES = ("drho", "dtheta", "dc", "dzl")


def grad_errors(got, ref, K_T):
    errs = {}
    for name, ax in CTRL_AXES.items():
        errs[name] = block_err(np.take(got[name], range(K_T), axis=ax), np.take(ref[name], range(K_T), axis=ax), ax)
    for name in TABLES:
        if ref[name] is None:
            continue
        errs[name] = block_err(got[name][None, None, :K_T], ref[name][None, None, :K_T], 1)
    return errs


def check_backward(name, inp, K_T, use_state=True, use_zl=True):
    B, L, K, P = inp["v"].shape
    m = inp["rho"].shape[1]
    log(f"{name}: backward B={B} L={L} K={K} K_T={K_T} m={m} P={P} io={inp['io']} "
        f"state={use_state} zero-lag={use_zl}")
    got = run_gpu_backward(inp, K_T, use_state, use_zl)
    ref = oracle_grads(inp, K_T, use_state, use_zl)
    errs = grad_errors(got, ref, K_T)
    log(f"{name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    tol = TOL[inp["io"]]
    for k, e in errs.items():
        bar = tol if k == "dv" else F32_GRAD_TOL
        assert e <= bar, f"{name}: {k} error {e:.3e} > {bar:.0e}"
    # channels k >= K_T are never written
    for nm, ax in CTRL_AXES.items():
        assert np.all(np.take(got[nm], range(K_T, K), axis=ax) == SENTINEL), nm
    for nm in TABLES:
        assert np.all(got[nm][K_T:] == SENTINEL), nm
    return errs


CASES = [
    # name, workload overrides, K_T, state, zero-lag
    ("tiny_f32_ragged", dict(index=0, L=37), 6, True, True),
    ("f32_m1_p32", dict(index=0, B=2, L=50, K=3, m=1, P=32), 3, True, False),
    ("f32_m2_p64_nostate", dict(index=0, B=2, L=70, K=3, m=2, P=64), 2, False, True),
    ("f32_m8_p128_two_slices", dict(index=0, B=2, L=45, K=3, m=8, P=128), 2, True, True),
    ("bf16_m4_p64", dict(index=1, B=2, L=300, K=4), 3, True, True),
    ("bf16_m8_p128", dict(index=2, B=2, L=200, K=3), 2, True, True),
    # one segment per sequence, seven sub-blocks each
    ("f32_single_segment", dict(index=0, B=16, L=100, K=128, m=1, P=16), 128, True, True),
    # eight segments of five sub-blocks, the last one shorter
    ("f32_multi_subblock_segments", dict(index=0, B=4, L=600, K=64, m=2, P=16), 64, True, True),
]


@pytest.mark.parametrize("name,over,K_T,use_state,use_zl", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(name, over, K_T, use_state, use_zl):
    idx = over.pop("index")
    w = I.workload(idx, **over)
    over["index"] = idx
    inp = I.make_backward_inputs(w)
    check_backward(name, inp, K_T, use_state, use_zl)


def test_backward_empty_sequence():
    """L = 0: the mode-table gradients are zero and dstate_in is dstate_out; B = 0 is a no-op.
    Empty arrays are passed as non-null dummies (every required pointer must be non-null)."""
    import torch
    from selective_spectral_ssm_amd import essh
    K, m, P, K_T = 3, 2, 16, 2
    dims = essh.make_dims(2, 0, K, m, P, K_T, 0, False, "f32")
    dummy = torch.zeros(64, device="cuda")
    tab = torch.rand((K, m), device="cuda") * 0.5 + 0.4
    c = torch.rand((K, m, 2), device="cuda")
    dso = torch.randn((2, K, m, 2, P), device="cuda")
    outs = [torch.full((K, m), SENTINEL, device="cuda"), torch.full((K, m), SENTINEL, device="cuda"),
            torch.full((K, m, 2), SENTINEL, device="cuda"), torch.full((K, m), SENTINEL, device="cuda")]
    dsi = torch.full_like(dso, SENTINEL)
    st = essh.essh_mixer_prefill_backward(dims, dummy, dummy, dummy, dummy, tab, tab, c, None, None, dummy, dso,
                                          dummy, dummy, dummy, dummy, *outs, dsi)
    assert st == essh.ESSH_OK, essh.status_string(st)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.all(o[:K_T] == 0) and torch.all(o[K_T:] == SENTINEL)
    assert torch.equal(dsi[:, :K_T], dso[:, :K_T]) and torch.all(dsi[:, K_T:] == SENTINEL)
    dims0 = essh.make_dims(0, 5, K, m, P, K_T, 0, False, "f32")
    assert essh.essh_mixer_prefill_backward(dims0, dummy, dummy, dummy, dummy, tab, tab, c, None, None, dummy,
                                            None, dummy, dummy, dummy, dummy, *outs, None) == essh.ESSH_OK
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# Full workload sizes, in the launch configuration bench.py times: sampled channels against
# the oracle run on those channels alone (channels are independent; the mode-table gradients
# of a channel sum over every batch row, so every row of a sampled channel is kept).
# ---------------------------------------------------------------------------

FULL = [(1, (0, 23)), (2, (0, 31)), (4, (23,))]


def _slice_channel(inp, k):
    out = dict(io=inp["io"])
    for key in ("v", "delta", "g_w", "g_r", "dy"):
        out[key] = inp[key][:, :, k:k + 1]
    for key in ("state_in", "dstate_out"):
        out[key] = inp[key][:, k:k + 1]
    for key in ("rho", "theta", "c", "zl"):
        out[key] = inp[key][k:k + 1]
    return out


@pytest.mark.parametrize("widx,chans", FULL, ids=[f"workload{w}" for w, _ in FULL])
def test_backward_full_size_sampled(widx, chans):
    w = I.workload(widx)
    K_T = w.K
    log(f"full-size backward: {w.name} B={w.B} L={w.L} K_T={K_T} sampled channels {chans}")
    inp = I.make_backward_inputs(w)
    got = run_gpu_backward(inp, K_T)
    for k in chans:
        ref = oracle_grads(_slice_channel(inp, k), 1)
        sub = {name: (np.take(got[name], [k], axis=CTRL_AXES[name]) if name in CTRL_AXES else got[name][k:k + 1])
               for name in list(CTRL_AXES) + list(TABLES)}
        errs = grad_errors(sub, ref, 1)
        log(f"{w.name} channel {k}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
        tol = TOL[inp["io"]]
        for n, e in errs.items():
            bar = tol if n == "dv" else F32_GRAD_TOL
            assert e <= bar, f"{w.name} channel {k}: {n} error {e:.3e} > {bar:.0e}"


def test_backward_graph_replay():
    """The backward call needs no zeroed workspace and enqueues no memset, so it can be captured
    in a HIP graph: three replays, with eager work and synchronisations between them, give the
    eager call's gradients bit for bit."""
    import torch
    from selective_spectral_ssm_amd import essh
    w = I.workload(1, B=2, L=300, K=6)
    inp = I.make_backward_inputs(w)
    d = {k: to_dev(inp[k]) for k in ("v", "delta", "g_w", "g_r", "rho", "theta", "c", "dy", "state_in", "dstate_out",
                                     "zl")}
    call = essh.PrefillBackward(d["v"], d["delta"], d["g_w"], d["g_r"], d["rho"], d["theta"], d["c"], d["dy"], K_T=5,
                                state_in=d["state_in"], dstate_out=d["dstate_out"], zl=d["zl"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call.stream = s
        call.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = {k: t.clone() for k, t in call.grads.items() if t is not None}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        call.run()
    for rep in range(3):
        for t in call.grads.values():
            if t is not None:
                t.zero_()                  # eager work between replays (channels past K_T stay zero)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, t in eager.items():
            assert torch.equal(call.grads[k], t), f"replay {rep}: {k} differs from the eager call"
