"""CPU oracle for the ESSH selective spectral mixer core -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or executes anything here, and
nothing here imports the product package.

Contents
  * ``prefill`` / ``decode_step``: the sequential recurrence of Eq. 5 / Eq. 9
    (paper "Elastic Selective Spectral Hybrids for Train-Once, Export-Many
    Budgeted Inference", Sec. 4.1 and App. B), written in plain C
    (``essh_oracle.c``) and run in float64.  A float32 build exists only for
    the CPU timing baseline.
  * ``reference``: independent NumPy restatements used to pin the C oracle
    (closed-form expansion Eq. 12, real 2xP damped-rotation form of Eq. 5,
    the chunk decomposition built on Eq. 6).

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, textbook special cases (FFT convolution, first-order IIR filtering)
and brute force; see the docstrings of those tests for the pin of each part.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "essh_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_lock = threading.Lock()
_libs = {}


def _so_path(prec: str) -> str:
    return os.path.join(_BUILD, f"libessh_oracle_{prec}.so")


def build(force: bool = False) -> None:
    """Compile the C oracle (float64 and float32 builds) with gcc."""
    os.makedirs(_BUILD, exist_ok=True)
    for prec, flags in (("f64", ["-DESSH_REAL=double", "-DESSH_SUFFIX=f64"]),
                        ("f32", ["-DESSH_REAL=float", "-DESSH_FLOAT", "-DESSH_SUFFIX=f32"])):
        out = _so_path(prec)
        if (not force and os.path.exists(out)
                and os.path.getmtime(out) >= os.path.getmtime(_SRC)):
            continue
        tmp = f"{out}.tmp{os.getpid()}"
        # -O2 without -ffast-math: the oracle keeps IEEE semantics.
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               *flags, _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)


def build_native(out_dir: str = None) -> str:
    """Compile the float32 build with -O3 -march=native for the host it runs on (the CPU
    timing baseline; the parity oracle stays the portable float64 build).  Returns its path."""
    out_dir = out_dir or _BUILD
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, "libessh_oracle_f32_native.so")
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = ["gcc", "-O3", "-march=native", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-DESSH_REAL=float", "-DESSH_FLOAT", "-DESSH_SUFFIX=f32", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(so_path: str, prec: str):
    lib = ctypes.CDLL(so_path)
    fn = getattr(lib, f"essh_oracle_prefill_{prec}")
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int] * 7 + [ctypes.c_void_p] * 11 + [ctypes.c_int]
    tu = getattr(lib, f"essh_oracle_threads_used_{prec}")
    tu.restype = ctypes.c_int
    return lib, fn, tu


def _lib(prec: str = "f64"):
    with _lock:
        if prec not in _libs:
            build()
            _libs[prec] = _bind(_so_path(prec), prec)
        return _libs[prec]


def _as(x, dt):
    return None if x is None else np.ascontiguousarray(x, dtype=dt)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def make_prefill(so_path=None, precision="f64"):
    """Return a ``prefill`` function bound to the oracle built at ``so_path``.

    The default binds the regular build.  Tests use other paths only to run
    the pins against deliberately broken copies of the oracle.
    """
    bound = None if so_path is None else _bind(so_path, precision)

    def prefill(v, delta, g_w, g_r, rho, theta, c, K_T=None, state_in=None,
                per_mode=None, y_out=None, nthreads=1, want_state=True, zl=None):
        """Run the sequential recurrence over all positions of v.

        Arguments are real arrays (already upcast from bf16 where relevant):
          v [B,L,K,P]; delta, g_w, g_r [B,L,K] (per channel) or [B,L,K,m] (per mode);
          rho, theta [K,m]; c [K,m,2]; state_in [B,K,m,2,P] or None (zero state);
          zl [K,m] zero-lag correction coefficients (Eq. 24) or None (core readout).
        ``y_out`` may be passed to observe that channels k >= K_T are left untouched.
        Returns (y, state_out) with y [B,L,K,P] and state_out [B,K,m,2,P]; channels
        k >= K_T of both keep their initial contents (zeros unless y_out is given).
        """
        dt = np.float64 if precision == "f64" else np.float32
        v = _as(v, dt)
        B, L, K, P = v.shape
        m = np.shape(rho)[1]
        pm = (np.ndim(delta) == 4) if per_mode is None else per_mode
        kt = K if K_T is None else int(K_T)
        delta_, g_w_, g_r_ = _as(delta, dt), _as(g_w, dt), _as(g_r, dt)
        rho_, theta_, c_, zl_ = _as(rho, dt), _as(theta, dt), _as(c, dt), _as(zl, dt)
        s_in = _as(state_in, dt)
        y = np.zeros((B, L, K, P), dt) if y_out is None else y_out
        assert y.dtype == dt and y.flags.c_contiguous and y.shape == (B, L, K, P)
        st = np.zeros((B, K, m, 2, P), dt) if want_state else None
        fn = (bound or _lib(precision))[1]
        rc = fn(B, L, K, m, P, kt, int(bool(pm)),
                _ptr(v), _ptr(delta_), _ptr(g_w_), _ptr(g_r_), _ptr(rho_), _ptr(theta_), _ptr(c_), _ptr(zl_),
                _ptr(s_in), _ptr(st), _ptr(y), int(nthreads))
        if rc != 0:
            raise RuntimeError(f"oracle prefill failed with code {rc}")
        return y, st

    return prefill


prefill = make_prefill()
prefill_f32 = make_prefill(precision="f32")


def threads_used(precision="f64", so_path=None) -> int:
    if so_path is not None:
        return _bind(so_path, precision)[2]()
    return _lib(precision)[2]()


def decode_step(state, v, delta, g_w, g_r, rho, theta, c, K_T=None, precision="f64", zl=None):
    """One token through n_layers independent mixers (decode is Eq. 5 for one position).

    state [NL,B,K,m,2,P] (not modified); v [NL,B,K,P]; delta, g_w, g_r [NL,B,K];
    rho, theta [NL,K,m]; c [NL,K,m,2]; zl [NL,K,m] or None (zero-lag correction, Eq. 24).
    Returns (y [NL,B,K,P], new_state).  Channels k >= K_T of the returned state keep
    their old values.
    """
    run = prefill if precision == "f64" else prefill_f32
    NL = v.shape[0]
    ys, sts = [], []
    for l in range(NL):
        y, st = run(v[l][:, None], delta[l][:, None], g_w[l][:, None], g_r[l][:, None],
                    rho[l], theta[l], c[l], K_T=K_T, state_in=state[l], zl=None if zl is None else zl[l])
        Kt = v.shape[2] if K_T is None else K_T
        st[:, Kt:] = state[l][:, Kt:]
        ys.append(y[:, 0])
        sts.append(st)
    return np.stack(ys), np.stack(sts)


from . import reference  # noqa: E402  (NumPy restatements used as pins)
