"""The C ABI library: it loads, exports what include/essh.h declares, and rejects bad
arguments on the host before anything is launched (runs without a GPU)."""
import ctypes
import os
import re

import pytest

from selective_spectral_ssm_amd import essh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "essh.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(essh.LIB_PATH):
        from selective_spectral_ssm_amd import build
        build.build(verbose=False)
    return essh.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(essh_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_set():
    assert declared_functions() == sorted(essh.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"libessh.so does not export {name}"
    assert lib.essh_abi_version() == 101


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert essh.status_string(code).startswith("ESSH_")


def test_decode_fused_validation(lib):
    """Host-side checks of the fused decode step: nothing is launched on these paths."""
    f = ctypes.c_void_p(FAKE)
    d = essh.make_dims(1, 1, 32, 8, 128, 32, 0)

    def call(n_layers=1, dims=d, d_model=4096, eps=1e-5, zl=None, u=f):
        return lib.essh_decode_fused_step(n_layers, ctypes.byref(dims), d_model, u, f, f, eps, f, f, f, f, f, zl, f,
                                          f, f, f, None)
    assert call(d_model=4100) == essh.ESSH_ERR_UNSUPPORTED          # not a multiple of 8
    assert call(d_model=8200) == essh.ESSH_ERR_UNSUPPORTED          # wider than the staged input
    assert call(eps=0.0) == essh.ESSH_ERR_INVALID_ARG
    assert call(eps=-1.0) == essh.ESSH_ERR_INVALID_ARG
    assert call(n_layers=0) == essh.ESSH_ERR_INVALID_ARG
    assert call(u=None) == essh.ESSH_ERR_INVALID_ARG
    wide = essh.make_dims(1, 1, 128, 8, 128, 128, 0)                # K_T P = 16384 > 8192
    assert call(dims=wide) == essh.ESSH_ERR_UNSUPPORTED
    bad_kt = essh.make_dims(1, 1, 32, 8, 128, 33, 0)
    assert call(dims=bad_kt) == essh.ESSH_ERR_INVALID_ARG
    assert lib.essh_decode_fused_step(1, ctypes.byref(d), 4096, f, ctypes.c_void_p(FAKE + 8), f, 1e-5, f, f, f, f,
                                      f, None, f, f, f, f, None) == essh.ESSH_ERR_INVALID_ARG   # weights misaligned


def test_noalloc_scratch_limit(lib):
    """The allocation-free prefill refuses, before launching anything, dims whose look-back
    records exceed its static scratch, and validates dims like the workspace entry point."""
    m = re.search(r"#define\s+ESSH_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == essh.NOALLOC_SCRATCH_BYTES
    p = [ctypes.c_void_p(FAKE)] * 7
    big = essh.make_dims(1, 131072, 24, 4, 64, 24, 128)
    assert essh.essh_prefill_workspace_bytes(big) > essh.NOALLOC_SCRATCH_BYTES
    assert lib.essh_mixer_prefill_noalloc(ctypes.byref(big), *p, None, None, None, ctypes.c_void_p(FAKE),
                                          None, None) == essh.ESSH_ERR_SCRATCH
    bad = essh.make_dims(1, 2048, 24, 4, 64, 25, 64)   # K_T > K
    assert lib.essh_mixer_prefill_noalloc(ctypes.byref(bad), *p, None, None, None, ctypes.c_void_p(FAKE),
                                          None, None) == essh.ESSH_ERR_INVALID_ARG
    fits = essh.make_dims(1, 131072, 24, 4, 64, 12, 128)
    assert 0 < essh.essh_prefill_workspace_bytes(fits) <= essh.NOALLOC_SCRATCH_BYTES


FAKE = 0x10000          # 16-byte-aligned stand-in address; never dereferenced on these error paths


def _call(dims, **over):
    p = {k: FAKE for k in ("v", "delta", "g_w", "g_r", "rho", "theta", "c", "y")}
    p["zl"] = None
    p.update(over)
    lib = essh.lib()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.essh_mixer_prefill(ctypes.byref(dims), vp(p["v"]), vp(p["delta"]), vp(p["g_w"]), vp(p["g_r"]),
                                  vp(p["rho"]), vp(p["theta"]), vp(p["c"]), vp(p["zl"]), None, None, vp(p["y"]),
                                  None, 0, None)


@pytest.mark.parametrize("field,value,code", [
    ("K_T", 0, essh.ESSH_ERR_INVALID_ARG),
    ("K_T", 25, essh.ESSH_ERR_INVALID_ARG),
    ("K", 0, essh.ESSH_ERR_INVALID_ARG),
    ("B", -1, essh.ESSH_ERR_INVALID_ARG),
    ("L", -5, essh.ESSH_ERR_INVALID_ARG),
    ("m", 3, essh.ESSH_ERR_UNSUPPORTED),
    ("m", 16, essh.ESSH_ERR_UNSUPPORTED),
    ("P", 48, essh.ESSH_ERR_UNSUPPORTED),
    ("P", 256, essh.ESSH_ERR_UNSUPPORTED),
    ("Lc", 16, essh.ESSH_ERR_UNSUPPORTED),
    ("io_dtype", 7, essh.ESSH_ERR_UNSUPPORTED),
    ("ctrl_per_mode", 2, essh.ESSH_ERR_INVALID_ARG),
])
def test_prefill_rejects_bad_dims(lib, field, value, code):
    d = essh.make_dims(8, 2048, 24, 4, 64, 24, 64)
    setattr(d, field, value)
    assert _call(d) == code


@pytest.mark.parametrize("which", ["v", "delta", "g_w", "g_r", "rho", "theta", "c", "y"])
def test_prefill_rejects_null_pointers(lib, which):
    d = essh.make_dims(8, 2048, 24, 4, 64, 24, 64)
    assert _call(d, **{which: None}) == essh.ESSH_ERR_INVALID_ARG


@pytest.mark.parametrize("which,addr", [("v", FAKE + 2), ("y", FAKE + 8), ("delta", FAKE + 2), ("g_w", FAKE + 1),
                                        ("zl", FAKE + 2)])
def test_prefill_rejects_misaligned(lib, which, addr):
    d = essh.make_dims(8, 2048, 24, 4, 64, 24, 64)
    assert _call(d, **{which: addr}) == essh.ESSH_ERR_INVALID_ARG


def test_decode_and_state_init_reject_bad_args(lib):
    d = essh.make_dims(1, 1, 32, 8, 128, 33, 0)
    f = ctypes.c_void_p(FAKE)
    assert lib.essh_mixer_decode_step(24, ctypes.byref(d), *([f] * 10), None) == essh.ESSH_ERR_INVALID_ARG
    d.K_T = 32
    assert lib.essh_mixer_decode_step(0, ctypes.byref(d), *([f] * 10), None) == essh.ESSH_ERR_INVALID_ARG
    assert lib.essh_mixer_decode_step(24, ctypes.byref(d), *([f] * 9), None, None) == essh.ESSH_ERR_INVALID_ARG
    assert lib.essh_mixer_decode_step(24, ctypes.byref(d), *([f] * 7), ctypes.c_void_p(FAKE + 2), f, f,
                                      None) == essh.ESSH_ERR_INVALID_ARG   # misaligned zl
    assert lib.essh_mixer_decode_step(65536, ctypes.byref(d), *([f] * 10), None) == essh.ESSH_ERR_UNSUPPORTED
    wide = essh.make_dims(65536, 1, 1, 1, 16, 1, 0)   # batch rows past the launch's grid extent
    assert lib.essh_mixer_decode_step(1, ctypes.byref(wide), *([f] * 10), None) == essh.ESSH_ERR_UNSUPPORTED
    assert lib.essh_state_init(None, 1, ctypes.byref(d), None) == essh.ESSH_ERR_INVALID_ARG
    assert lib.essh_state_init(ctypes.c_void_p(FAKE + 4), 1, ctypes.byref(d), None) == essh.ESSH_ERR_INVALID_ARG
    assert lib.essh_mixer_prefill(None, *([f] * 12), 0, None) == essh.ESSH_ERR_INVALID_ARG


def test_workspace_query_is_total(lib):
    for args in [(8, 2048, 24, 4, 64, 24, 64), (16, 2048, 32, 8, 128, 8, 64), (1, 131072, 24, 4, 64, 6, 128)]:
        d = essh.make_dims(*args)
        assert essh.essh_prefill_workspace_bytes(d) >= 0
    d = essh.make_dims(8, 2048, 24, 3, 64, 24, 64)   # unsupported m -> 0
    assert essh.essh_prefill_workspace_bytes(d) == 0


def _call_ws(dims, ws, ws_bytes):
    p = [ctypes.c_void_p(FAKE)] * 7
    lib = essh.lib()
    return lib.essh_mixer_prefill(ctypes.byref(dims), *p, None, None, None, ctypes.c_void_p(FAKE),
                                  None if ws is None else ctypes.c_void_p(ws), ws_bytes, None)


def test_segmented_prefill_needs_a_workspace(lib):
    """Few (batch row, channel) sequences -> the scan is segmented and needs look-back space:
    at least the aggregate and inclusive states (2 x 2m x P fp32) of every segment, and at most
    that for one segment per chunk plus a channel-major copy of the controls (8 bytes per
    position and sequence)."""
    d = essh.make_dims(1, 131072, 24, 4, 64, 6, 128)
    need = essh.essh_prefill_workspace_bytes(d)
    nchunks = 131072 // 128
    assert need >= 2 * (1 * 6) * 2 * 2 * 4 * 64 * 4          # at least two segments per sequence
    assert need <= 2 * (1 * 6) * nchunks * 2 * 4 * 64 * 4 + 2 * 6 * nchunks * 64 + 6 * 131072 * 8 + 4096
    assert _call_ws(d, None, 0) == essh.ESSH_ERR_WORKSPACE
    assert _call_ws(d, FAKE * 16, need - 1) == essh.ESSH_ERR_WORKSPACE
    assert _call_ws(d, FAKE * 16 + 16, need) == essh.ESSH_ERR_WORKSPACE     # not 256-byte aligned


def _call_bwd(dims, ws=FAKE * 16, ws_bytes=None, **over):
    names = ("v", "delta", "g_w", "g_r", "rho", "theta", "c", "zl", "state_in", "dy", "dstate_out", "dv", "ddelta",
             "dg_w", "dg_r", "drho", "dtheta", "dc", "dzl", "dstate_in")
    p = {k: FAKE for k in names}
    for k in ("zl", "state_in", "dstate_out", "dzl", "dstate_in"):
        p[k] = None
    p.update(over)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    if ws_bytes is None:
        ws_bytes = essh.essh_prefill_backward_workspace_bytes(dims)
    return essh.lib().essh_mixer_prefill_backward(ctypes.byref(dims), *[vp(p[k]) for k in names], vp(ws), ws_bytes,
                                                  None)


def test_backward_validation(lib):
    """Host-side checks of the backward entry point: nothing is launched on these paths."""
    d = essh.make_dims(8, 2048, 24, 4, 64, 24, 0)
    need = essh.essh_prefill_backward_workspace_bytes(d)
    assert need > 0
    pm = essh.make_dims(8, 2048, 24, 4, 64, 24, 0, per_mode=True)
    assert essh.essh_prefill_backward_workspace_bytes(pm) == 0
    assert _call_bwd(pm, ws_bytes=need) == essh.ESSH_ERR_UNSUPPORTED                 # per-mode controls
    for name in ("v", "delta", "g_w", "g_r", "rho", "theta", "c", "dy", "dv", "ddelta", "dg_w", "dg_r", "drho",
                 "dtheta", "dc"):
        assert _call_bwd(d, **{name: None}) == essh.ESSH_ERR_INVALID_ARG, name       # required pointers
    for name, addr in (("v", FAKE + 2), ("dy", FAKE + 8), ("dv", FAKE + 4), ("ddelta", FAKE + 2),
                       ("dstate_in", FAKE + 2), ("zl", FAKE + 1)):
        assert _call_bwd(d, **{name: addr}) == essh.ESSH_ERR_INVALID_ARG, name       # misaligned
    assert _call_bwd(d, ws=None) == essh.ESSH_ERR_WORKSPACE
    assert _call_bwd(d, ws_bytes=need - 1) == essh.ESSH_ERR_WORKSPACE
    assert _call_bwd(d, ws=FAKE * 16 + 16) == essh.ESSH_ERR_WORKSPACE                # not 256-byte aligned
    bad = essh.make_dims(8, 2048, 24, 4, 64, 25, 0)
    assert _call_bwd(bad, ws_bytes=need) == essh.ESSH_ERR_INVALID_ARG                # K_T > K
    wide = essh.make_dims(4096, 16, 32, 4, 64, 32, 0)                                 # B K_T > 65535
    assert _call_bwd(wide) == essh.ESSH_ERR_UNSUPPORTED
    odd = essh.make_dims(8, 2048, 24, 3, 64, 24, 0)
    assert _call_bwd(odd, ws_bytes=need) == essh.ESSH_ERR_UNSUPPORTED                # m outside the set


def test_backward_workspace_covers_its_arrays(lib):
    """The workspace holds at least the state checkpoints (2 m P fp32 per 16 positions and
    sequence), the channel-major controls and the control gradients (16 bytes per position and
    sequence each, per column slice for the gradients)."""
    for B, L, K, m, P in [(8, 2048, 24, 4, 64), (16, 2048, 32, 8, 128), (1, 131072, 24, 4, 64), (2, 37, 3, 2, 16)]:
        d = essh.make_dims(B, L, K, m, P, K, 0)
        need = essh.essh_prefill_backward_workspace_bytes(d)
        nseq = B * K
        slices = P // 32 if (m == 8 and P >= 64) else max(1, P // 64)
        ck = nseq * ((L + 15) // 16) * 2 * m * P * 4
        assert need >= ck + nseq * L * 16 * (1 + slices), (B, L, K, m, P)
