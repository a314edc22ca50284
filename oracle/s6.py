"""fp64 Mamba-1 selective scan (S6), the second member of the family.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Definition followed: Sasha Rush, "Mamba: The Hard Way", Part 5 ("Mamba /
S6"). The continuous-time parameters are discretized per step,

    a_[n, d, t] = exp(delta[d, t] * A[d, n]),   b_[n, d, t] = B[n, t] * delta[d, t]

and the scan runs one scalar state per (state n, channel d):

    h[n, d] <- a_[n, d, t] * h[n, d] + b_[n, d, t] * x[d, t]
    y[d, t]  = sum_n C[n, t] * h[n, d]

as the page's plain PyTorch loop does (its batched version adds the batch
dimension in front). Readings taken here:

* A is one [channels, dstate] matrix shared by every batch row (the page's
  test tensor is a constant, the same for every row; the Mamba reference
  kernel it compares against takes A without a batch dimension).
* No skip term and no gate: the page runs the scan with neither.
* ``h0`` is an optional initial state [batch, channels, dstate] (zeros when
  None); the scan also returns the final state, so calls can be chained.

Layouts (the page's tensor shapes without their singleton dimensions):
x, delta, y [batch, channels, seqlen]; B, C [batch, dstate, seqlen];
A [channels, dstate].
"""
from __future__ import annotations

import numpy as np


def s6_sequential(x, delta, A, B, C, h0=None):
    """Run the scan token by token in float64.

    Returns ``(y, h_final)``: y [batch, channels, seqlen] and the state after
    the last token [batch, channels, dstate].
    """
    x = np.asarray(x, dtype=np.float64)
    delta = np.asarray(delta, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    bt, D, L = x.shape
    N = A.shape[1]
    h = np.zeros((bt, D, N)) if h0 is None else np.array(h0, dtype=np.float64, copy=True)
    y = np.zeros((bt, D, L))
    for t in range(L):
        a_ = np.exp(delta[:, :, t, None] * A[None, :, :])          # [bt, D, N]
        b_ = B[:, None, :, t] * delta[:, :, t, None]               # [bt, D, N]
        h = a_ * h + b_ * x[:, :, t, None]
        y[:, :, t] = np.einsum("bdn,bn->bd", h, C[:, :, t])
    return y, h
