"""Python binding of libessh (C ABI in include/essh.h).

Argument marshalling only: tensors are passed to the library as raw device
pointers, with the current HIP stream, and every step of the computation runs
in the library's HIP kernels.  PyTorch supplies device memory and streams.

The library is loaded on first use.  If it has not been built this module
raises ``EsshLibraryMissing``: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libessh.so")

ESSH_OK, ESSH_ERR_INVALID_ARG, ESSH_ERR_UNSUPPORTED, ESSH_ERR_WORKSPACE, ESSH_ERR_HIP = 0, -1, -2, -3, -4
ESSH_ERR_SCRATCH = -5
NOALLOC_SCRATCH_BYTES = 32 << 20
ESSH_F32, ESSH_BF16 = 0, 1

# Every symbol the C header declares (checked by the tests against include/essh.h).
EXPORTED = ("essh_abi_version", "essh_status_string", "essh_state_init",
            "essh_prefill_workspace_bytes", "essh_mixer_prefill", "essh_mixer_prefill_noalloc",
            "essh_mixer_decode_step", "essh_decode_fused_step", "essh_prefill_backward_workspace_bytes",
            "essh_mixer_prefill_backward")


class EsshLibraryMissing(RuntimeError):
    pass


class EsshError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class EsshScanError(RuntimeError):
    """A segmented prefill reported an error in its workspace (header word 1): that call's
    outputs are invalid.  Bit 1: a bounded look-back wait ran out; bit 2: more tickets than
    workgroups (a workspace that was not zero-filled before its first use)."""

    def __init__(self, bits: int):
        self.bits = bits
        super().__init__(f"segmented prefill scan error bits 0x{bits:x} (outputs of that call are invalid)")


# Byte offset and size of the error word in a prefill workspace (include/essh.h).
SCAN_ERROR_OFFSET = 4


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("L", ctypes.c_int32), ("K", ctypes.c_int32),
                ("m", ctypes.c_int32), ("P", ctypes.c_int32), ("K_T", ctypes.c_int32),
                ("Lc", ctypes.c_int32), ("ctrl_per_mode", ctypes.c_int32), ("io_dtype", ctypes.c_int32)]


_lib = None


def lib():
    """Load libessh.so (once)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise EsshLibraryMissing(
                f"{LIB_PATH} is not built; run `python -m selective_spectral_ssm_amd.build` "
                "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.essh_abi_version.restype = I32
        L.essh_abi_version.argtypes = []
        L.essh_status_string.restype = ctypes.c_char_p
        L.essh_status_string.argtypes = [ctypes.c_int]
        L.essh_state_init.restype = ctypes.c_int
        L.essh_state_init.argtypes = [P, I32, ctypes.POINTER(Dims), P]
        L.essh_prefill_workspace_bytes.restype = SZ
        L.essh_prefill_workspace_bytes.argtypes = [ctypes.POINTER(Dims)]
        L.essh_mixer_prefill.restype = ctypes.c_int
        L.essh_mixer_prefill.argtypes = [ctypes.POINTER(Dims)] + [P] * 12 + [SZ, P]
        L.essh_mixer_prefill_noalloc.restype = ctypes.c_int
        L.essh_mixer_prefill_noalloc.argtypes = [ctypes.POINTER(Dims)] + [P] * 13
        L.essh_decode_fused_step.restype = ctypes.c_int
        L.essh_decode_fused_step.argtypes = ([I32, ctypes.POINTER(Dims), I32] + [P] * 3 + [ctypes.c_float]
                                             + [P] * 11)
        L.essh_mixer_decode_step.restype = ctypes.c_int
        L.essh_mixer_decode_step.argtypes = [I32, ctypes.POINTER(Dims)] + [P] * 10 + [P]
        L.essh_prefill_backward_workspace_bytes.restype = SZ
        L.essh_prefill_backward_workspace_bytes.argtypes = [ctypes.POINTER(Dims)]
        L.essh_mixer_prefill_backward.restype = ctypes.c_int
        L.essh_mixer_prefill_backward.argtypes = [ctypes.POINTER(Dims)] + [P] * 21 + [SZ, P]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().essh_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libessh must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ESSH_BF16
    if t.dtype == torch.float32:
        return ESSH_F32
    raise TypeError(f"io dtype must be bfloat16 or float32, got {t.dtype}")


def _check(status: int, what: str):
    if status != ESSH_OK:
        raise EsshError(status, what)


def make_dims(B, L, K, m, P, K_T=None, Lc=0, per_mode=False, io="bf16") -> Dims:
    return Dims(int(B), int(L), int(K), int(m), int(P), int(K if K_T is None else K_T), int(Lc),
                int(bool(per_mode)), ESSH_BF16 if io in ("bf16", torch.bfloat16, ESSH_BF16) else ESSH_F32)


# ---------------------------------------------------------------------------
# Raw entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def essh_state_init(state: torch.Tensor, n_layers: int, dims: Dims, stream=None) -> None:
    _check(lib().essh_state_init(_ptr(state), int(n_layers), ctypes.byref(dims), _stream(stream)),
           "essh_state_init")


def essh_prefill_workspace_bytes(dims: Dims) -> int:
    return int(lib().essh_prefill_workspace_bytes(ctypes.byref(dims)))


def essh_mixer_prefill(dims: Dims, v, delta, g_w, g_r, rho, theta, c, zl, state_in, state_out, y,
                       workspace=None, workspace_bytes: int = 0, stream=None) -> int:
    """Direct call; returns the status code (no exception) so tests can check error paths."""
    return lib().essh_mixer_prefill(ctypes.byref(dims), _ptr(v), _ptr(delta), _ptr(g_w), _ptr(g_r),
                                    _ptr(rho), _ptr(theta), _ptr(c), _ptr(zl), _ptr(state_in), _ptr(state_out),
                                    _ptr(y), _ptr(workspace), int(workspace_bytes), _stream(stream))


def essh_mixer_prefill_noalloc(dims: Dims, v, delta, g_w, g_r, rho, theta, c, zl, state_in, state_out, y,
                               scan_error=None, stream=None) -> int:
    """Direct call of the allocation-free prefill; returns the status code."""
    return lib().essh_mixer_prefill_noalloc(ctypes.byref(dims), _ptr(v), _ptr(delta), _ptr(g_w), _ptr(g_r),
                                            _ptr(rho), _ptr(theta), _ptr(c), _ptr(zl), _ptr(state_in),
                                            _ptr(state_out), _ptr(y), _ptr(scan_error), _stream(stream))


def essh_decode_fused_step(n_layers: int, dims: Dims, d_model: int, u, w_in, beta, eps_norm: float, w_ctl, b_ctl,
                           rho, theta, c, zl, w_out, state, z, y, stream=None) -> int:
    """Direct call of the fused decode step with projections; returns the status code."""
    return lib().essh_decode_fused_step(int(n_layers), ctypes.byref(dims), int(d_model), _ptr(u), _ptr(w_in),
                                        _ptr(beta), float(eps_norm), _ptr(w_ctl), _ptr(b_ctl), _ptr(rho),
                                        _ptr(theta), _ptr(c), _ptr(zl), _ptr(w_out), _ptr(state), _ptr(z), _ptr(y),
                                        _stream(stream))


def essh_mixer_decode_step(n_layers: int, dims: Dims, v, delta, g_w, g_r, rho, theta, c, zl, state, y,
                           stream=None) -> int:
    return lib().essh_mixer_decode_step(int(n_layers), ctypes.byref(dims), _ptr(v), _ptr(delta), _ptr(g_w),
                                        _ptr(g_r), _ptr(rho), _ptr(theta), _ptr(c), _ptr(zl), _ptr(state), _ptr(y),
                                        _stream(stream))


def essh_prefill_backward_workspace_bytes(dims: Dims) -> int:
    return int(lib().essh_prefill_backward_workspace_bytes(ctypes.byref(dims)))


def essh_mixer_prefill_backward(dims: Dims, v, delta, g_w, g_r, rho, theta, c, zl, state_in, dy, dstate_out,
                                dv, ddelta, dg_w, dg_r, drho, dtheta, dc, dzl, dstate_in,
                                workspace=None, workspace_bytes: int = 0, stream=None) -> int:
    """Direct call of the prefill's backward pass; returns the status code."""
    return lib().essh_mixer_prefill_backward(
        ctypes.byref(dims), _ptr(v), _ptr(delta), _ptr(g_w), _ptr(g_r), _ptr(rho), _ptr(theta), _ptr(c), _ptr(zl),
        _ptr(state_in), _ptr(dy), _ptr(dstate_out), _ptr(dv), _ptr(ddelta), _ptr(dg_w), _ptr(dg_r), _ptr(drho),
        _ptr(dtheta), _ptr(dc), _ptr(dzl), _ptr(dstate_in), _ptr(workspace), int(workspace_bytes),
        _stream(stream))


# ---------------------------------------------------------------------------
# Tensor-level helpers
# ---------------------------------------------------------------------------

class Prefill:
    """A prepared prefill call: dims, workspace and output buffers for fixed shapes.

    ``run`` only enqueues the library call, so it can be timed or captured in
    a HIP graph.
    """

    def __init__(self, v, delta, g_w, g_r, rho, theta, c, K_T=None, Lc=0,
                 state_in=None, want_state=True, y=None, stream=None, zl=None):
        B, L, K, P = v.shape
        m = rho.shape[1]
        per_mode = delta.dim() == 4
        self.dims = make_dims(B, L, K, m, P, K_T, Lc, per_mode, "bf16" if v.dtype == torch.bfloat16 else "f32")
        self.args = (v, delta, g_w, g_r, rho, theta, c, zl)
        self.state_in = state_in
        self.y = y if y is not None else torch.empty_like(v)
        self.state_out = (torch.zeros((B, K, m, 2, P), dtype=torch.float32, device=v.device)
                          if want_state else None)
        ws = essh_prefill_workspace_bytes(self.dims)
        # zero-filled once: the library keeps the look-back header armed across calls
        self.workspace = torch.zeros(max(ws, 1), dtype=torch.uint8, device=v.device) if ws else None
        self.ws_bytes = ws
        self.stream = stream

    def run(self):
        st = essh_mixer_prefill(self.dims, *self.args, self.state_in, self.state_out, self.y,
                                self.workspace, self.ws_bytes, self.stream)
        _check(st, "essh_mixer_prefill")
        return self.y, self.state_out

    def check(self):
        """Synchronise and raise EsshScanError if any call so far set the workspace error word.

        The word is sticky (the library never clears it), so one check after a batch of
        calls covers all of them; it is cleared here after being reported."""
        check_workspace(self.workspace)


def check_workspace(workspace) -> None:
    """Raise EsshScanError if the error word of a prefill workspace is set, and clear it."""
    if workspace is None:
        return
    word = workspace[SCAN_ERROR_OFFSET:SCAN_ERROR_OFFSET + 4]
    bits = int(word.view(torch.int32).item())   # synchronises with the device
    if bits:
        word.zero_()
        raise EsshScanError(bits)


def prefill(v, delta, g_w, g_r, rho, theta, c, K_T=None, Lc=0, state_in=None, want_state=True, y=None, zl=None):
    """Chunked prefill of one mixer (zl: zero-lag coefficients or None).  Returns (y, state_out or None).

    Synchronises with the device when the call needed a workspace, to check its error word."""
    call = Prefill(v, delta, g_w, g_r, rho, theta, c, K_T, Lc, state_in, want_state, y, zl=zl)
    out = call.run()
    call.check()
    return out


class PrefillBackward:
    """A prepared backward call: dims, workspace and gradient buffers for fixed shapes.

    Gradients of channels k >= K_T are left at zero (the library never writes them).  ``run``
    only enqueues the library call."""

    def __init__(self, v, delta, g_w, g_r, rho, theta, c, dy, K_T=None, state_in=None, dstate_out=None,
                 zl=None, want_dzl=None, want_dstate_in=True, stream=None):
        B, L, K, P = v.shape
        m = rho.shape[1]
        dev = v.device
        self.dims = make_dims(B, L, K, m, P, K_T, 0, delta.dim() == 4, "bf16" if v.dtype == torch.bfloat16 else "f32")
        self.args = (v, delta, g_w, g_r, rho, theta, c, zl, state_in, dy, dstate_out)
        f32 = dict(dtype=torch.float32, device=dev)
        self.grads = dict(
            dv=torch.zeros_like(v), ddelta=torch.zeros(delta.shape, **f32), dg_w=torch.zeros(g_w.shape, **f32),
            dg_r=torch.zeros(g_r.shape, **f32), drho=torch.zeros(rho.shape, **f32),
            dtheta=torch.zeros(theta.shape, **f32), dc=torch.zeros(c.shape, **f32),
            dzl=torch.zeros(rho.shape, **f32) if (zl is not None if want_dzl is None else want_dzl) else None,
            dstate_in=torch.zeros((B, K, m, 2, P), **f32) if want_dstate_in else None)
        self.ws_bytes = essh_prefill_backward_workspace_bytes(self.dims)
        self.workspace = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=dev) if self.ws_bytes else None
        self.stream = stream

    def run(self):
        g = self.grads
        st = essh_mixer_prefill_backward(self.dims, *self.args, g["dv"], g["ddelta"], g["dg_w"], g["dg_r"],
                                         g["drho"], g["dtheta"], g["dc"], g["dzl"], g["dstate_in"],
                                         self.workspace, self.ws_bytes, self.stream)
        _check(st, "essh_mixer_prefill_backward")
        return g


def prefill_backward(v, delta, g_w, g_r, rho, theta, c, dy, K_T=None, state_in=None, dstate_out=None, zl=None):
    """Gradients of the prefill for dL/dy = dy (and dL/dstate_out = dstate_out).  Returns a dict
    dv, ddelta, dg_w, dg_r, drho, dtheta, dc, dzl (None without zl), dstate_in."""
    return PrefillBackward(v, delta, g_w, g_r, rho, theta, c, dy, K_T, state_in, dstate_out, zl).run()


def decode_step(state, v, delta, g_w, g_r, rho, theta, c, K_T=None, y=None, zl=None):
    """One token through n_layers mixers; state [NL,B,K,m,2,P] is updated in place.  Returns y."""
    NL, B, K, P = v.shape
    m = rho.shape[-1]
    dims = make_dims(B, 1, K, m, P, K_T, 0, delta.dim() == 4, "bf16" if v.dtype == torch.bfloat16 else "f32")
    if y is None:
        y = torch.empty_like(v)
    _check(essh_mixer_decode_step(NL, dims, v, delta, g_w, g_r, rho, theta, c, zl, state, y),
           "essh_mixer_decode_step")
    return y
