"""One token of the Mamba-2 SSD recurrence in fp64: the decode step.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Definition followed (NVIDIA developer blog, "Accelerating Mamba-2 with
high-performance forward-pass kernels in NVIDIA CUDA Tile", section
"Mamba-2 architecture", the core recurrence): for one new token of every
sequence b and every head h, with g the head's group,

    alpha        = exp(A[h] * dt[b, h])
    state[p, n] <- alpha * state[p, n] + dt[b, h] * x[b, h, p] * B[b, g, n]
    y[b, h, p]   = sum_n C[b, g, n] * state[p, n] + D[h] * x[b, h, p]

with y reading the updated state and the state stored headdim-major
(``[p, n]``), the readings ``ssd_seq.py`` states. Written per (b, h) with
explicit outer and inner products, not through ``ssd_sequential``; the pins
in ``tests/test_oracle_pins.py`` chain it over whole sequences and compare
with both forward oracles and with every forward pin.
"""
from __future__ import annotations

import numpy as np


def ssd_step(x, dt, A, B, C, D, state):
    """Advance every (sequence, head) by one token, in float64.

    Args:
      x:  [batch, nheads, headdim]
      dt: [batch, nheads]
      A, D: [nheads]
      B, C: [batch, ngroups, dstate]
      state: [batch, nheads, headdim, dstate] (not modified)

    Returns ``(y, new_state)``: y ``[batch, nheads, headdim]`` and the updated
    state, both float64.
    """
    x = np.asarray(x, dtype=np.float64)
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    state = np.asarray(state, dtype=np.float64)
    bt, H, P = x.shape
    G = B.shape[1]
    if H % G:
        raise ValueError("nheads must be a multiple of ngroups")
    per_group = H // G
    new_state = np.empty_like(state)
    y = np.empty((bt, H, P))
    for b in range(bt):
        for h in range(H):
            g = h // per_group
            alpha = np.exp(A[h] * dt[b, h])
            upd = np.outer(x[b, h], B[b, g]) * dt[b, h]          # dt x B^T, [P, N]
            s = alpha * state[b, h] + upd
            new_state[b, h] = s
            y[b, h] = s @ C[b, g] + D[h] * x[b, h]
    return y, new_state
