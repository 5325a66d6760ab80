"""Planted mistakes in the oracle must be caught by the pins (CPU only).

Each mutant is a copy of oracle/essh_oracle.c with one plausible mistake
(a dropped term, a wrong sign, a wrong index, a conjugated coefficient, ...),
compiled into a temporary library.  The pins of tests/oracle_pins.py are run
against it and at least one of them must fail.  The regular oracle is never
modified.
"""
import os
import subprocess

import pytest

import oracle
from tests.oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "essh_oracle.c")

# (name, original text, replacement)
MUTANTS = [
    ("clock_sign", "R_EXP(-delta[ci])", "R_EXP(delta[ci] * 0.0)"),
    ("rotation_conjugated", "(R_COS(th) + I * R_SIN(th))", "(R_COS(th) - I * R_SIN(th))"),
    ("readout_conjugated", "c[((size_t)k * m + j) * 2] + I * c[((size_t)k * m + j) * 2 + 1]",
     "c[((size_t)k * m + j) * 2] - I * c[((size_t)k * m + j) * 2 + 1]"),
    ("write_gate_dropped", "lam * h[(size_t)j * P + p] + gw * vt[p]", "lam * h[(size_t)j * P + p] + vt[p]"),
    ("read_gate_dropped", "acc[p] += gr * C_RE(cc * hn);", "acc[p] += C_RE(cc * hn);"),
    ("readout_before_update", "h[(size_t)j * P + p] = hn;\n                        acc[p] += gr * C_RE(cc * hn);",
     "acc[p] += gr * C_RE(cc * h[(size_t)j * P + p]);\n                        h[(size_t)j * P + p] = hn;"),
    ("rho_index_transposed", "real rk = rho[(size_t)k * m + j];", "real rk = rho[(size_t)j * K + k];"),
    ("clock_on_injection", "cplx hn = lam * h[(size_t)j * P + p] + gw * vt[p];",
     "cplx hn = lam * (h[(size_t)j * P + p] + gw * vt[p]);"),
    ("state_imag_plane_swapped", "state_out[s + P + p] = C_IM(hv);", "state_out[s + P + p] = -C_IM(hv);"),
    ("state_in_imag_dropped", "h0 = state_in[s + p] + I * state_in[s + P + p];", "h0 = state_in[s + p];"),
    ("per_mode_index", "size_t ci = per_mode ? row * m + j : row;", "size_t ci = per_mode ? row * m : row;"),
    ("imag_readout_dropped", "acc[p] += gr * C_RE(cc * hn);", "acc[p] += gr * C_RE(cc) * C_RE(hn);"),
    ("zero_lag_sign", "acc[p] -= zc * vt[p];", "acc[p] += zc * vt[p];"),
    ("zero_lag_read_gate_dropped", "real zc = zl[(size_t)k * m + j] * gr * gw", "real zc = zl[(size_t)k * m + j] * gw"),
    ("zero_lag_imag_part", "* gr * gw * c[((size_t)k * m + j) * 2];", "* gr * gw * c[((size_t)k * m + j) * 2 + 1];"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutant {name}: anchor text not found exactly once"
    path = tmp_path / f"mut_{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"libmut_{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-DESSH_REAL=double", "-DESSH_SUFFIX=f64", str(path), "-o", str(so), "-lm"],
                   check=True)
    return str(so)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    prefill = oracle.make_prefill(_build_mutant(tmp_path, name, old, new))
    failed = []
    for pname, pin, kw in ALL_PINS:
        try:
            err, tol = pin(prefill, **kw)
        except Exception:  # a crash or NaN-induced failure also counts as caught
            failed.append(pname)
            continue
        if not err <= tol:
            failed.append(pname)
    assert failed, f"planted mistake '{name}' passed every pin"
