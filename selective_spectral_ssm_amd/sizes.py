"""Size and work accounting for the selective mixer core (host-side arithmetic only).

State: each retained channel carries m complex mode states of P values, i.e.
2 K_T m P real entries per spectral layer (ESSH paper, Sec. 4.3), kept in fp32.

Algorithmic work is what the method must move or compute, excluding any
workspace, re-reads or padding of an implementation:

  prefill, per (token, retained channel):
      bytes = P*s_io (v) + P*s_io (y) + 4 (clock) + 2*s_io (write and read gate)
      flops = 10*m*P + 2*P   (per mode and value: complex state update 7,
                              readout 3; per value: write-gate and read-gate
                              products)
    plus, per call, the mode tables (16 B per retained (k, j): rho, theta, c)
    and the final state if it is written (8 B per retained (b, k, j, p)).

  decode, per (layer, batch row, retained channel):
      bytes = 2 * 8*m*P (state read + written, fp32 complex)
              + P*s_io (v) + P*s_io (y) + 4 + 2*s_io (clock, gates)
              + 16*m (mode tables)
      flops = 10*m*P + 2*P

  prefill backward, per (token, retained channel):
      bytes = 3*P*s_io (v and dy read, dv written) + 4 + 2*s_io (clock, gates read)
              + 3*4 (ddelta, dg_w, dg_r written, fp32)
    plus, per call, the mode tables read (16 B per retained (k, j), 20 with zero-lag
    coefficients) and their gradients written (same), and the entering state, the final
    state's gradient and dstate_in (8 B each per retained (b, k, j, p)).
"""
from __future__ import annotations

IO_BYTES = {"f32": 4, "bf16": 2}


def state_bytes(n_layers: int, B: int, K: int, m: int, P: int) -> int:
    """Bytes of fp32 recurrent state for K retained channels over n_layers layers."""
    return 2 * n_layers * B * K * m * P * 4


def prefill_bytes(B: int, L: int, K_T: int, m: int, P: int, io: str,
                  write_state: bool = False, per_mode: bool = False) -> int:
    s = IO_BYTES[io]
    nc = m if per_mode else 1
    per_tok = 2 * P * s + nc * (4 + 2 * s)
    total = B * L * K_T * per_tok + K_T * m * 16
    if write_state:
        total += state_bytes(1, B, K_T, m, P)
    return total


def prefill_flops(B: int, L: int, K_T: int, m: int, P: int) -> int:
    return B * L * K_T * (10 * m * P + 2 * P)


def decode_bytes(n_layers: int, B: int, K_T: int, m: int, P: int, io: str) -> int:
    s = IO_BYTES[io]
    per = 2 * 8 * m * P + 2 * P * s + 4 + 2 * s + 16 * m
    return n_layers * B * K_T * per


def decode_fused_bytes(n_layers: int, B: int, K_T: int, m: int, P: int, d_model: int, io: str,
                       zero_lag: bool = False) -> int:
    """Fused decode step with projections: the retained rows of W_in (K_T P x d) and of the gate
    and clock projections (3 K_T m x d) and the first K_T P columns of W_out, all bf16, their
    biases and blend coefficients, the modal tables; per batch row u, the state read and
    written, z and y (fp32)."""
    s = IO_BYTES[io]
    weights = 2 * d_model * (2 * K_T * P + 3 * K_T * m) + 4 * (3 * K_T * m + K_T) + K_T * m * (16 + (4 if zero_lag else 0))
    per_row = d_model * s + 2 * 8 * K_T * m * P + 4 * K_T * P + 4 * d_model
    return n_layers * (weights + B * per_row)


def decode_fused_flops(n_layers: int, B: int, K_T: int, m: int, P: int, d_model: int) -> int:
    return n_layers * B * (2 * d_model * (2 * K_T * P + 3 * K_T * m) + K_T * (10 * m * P + 2 * P))


def decode_flops(n_layers: int, B: int, K_T: int, m: int, P: int) -> int:
    return n_layers * B * K_T * (10 * m * P + 2 * P)


def backward_bytes(B: int, L: int, K_T: int, m: int, P: int, io: str, zero_lag: bool = True,
                   states: bool = True) -> int:
    s = IO_BYTES[io]
    per_tok = 3 * P * s + 4 + 2 * s + 12
    tab = K_T * m * (20 if zero_lag else 16)
    total = B * L * K_T * per_tok + 2 * tab
    if states:
        total += 3 * state_bytes(1, B, K_T, m, P)
    return total
