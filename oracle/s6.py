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


def s6_bwd_sequential(x, delta, A, B, C, dy, h0=None, dhT=None):
    """Every input's gradient of the scan above, by reverse mode through the
    token recurrence in float64, for a loss whose gradients with respect to
    the outputs are ``dy`` (like y) and ``dhT`` (like the final state; None
    means zero).

    The state's adjoint runs the same scan backwards in time ("Mamba: The
    Hard Way", Part 3, applied to each scalar chain of Part 5): with
    a_t = exp(delta_t A) and u_t = B_t delta_t x_t,

        g_t = C_t dy_t + a_{t+1} g_{t+1}          (g after the last token: dhT)

    and then, per step, from h_t = a_t h_{t-1} + u_t and y_t = sum_n C_t h_t:

        dx_t     = sum_n g_t B_t delta_t
        ddelta_t = sum_n g_t (A a_t h_{t-1} + B_t x_t)
        dA       = sum_t g_t delta_t a_t h_{t-1}        (summed over batch rows)
        dB_t     = sum_d g_t delta_t x_t                (summed over channels)
        dC_t     = sum_d dy_t h_t
        dh0      = a_0 g_0

    Returns a dict with dx, ddelta (like x), dA (like A), dB, dC (like B) and
    dh0 (like h0 when h0 is given, else the gradient at a zero initial state).
    """
    x = np.asarray(x, dtype=np.float64)
    delta = np.asarray(delta, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    bt, D, L = x.shape
    N = A.shape[1]
    # forward, keeping every state: hs[t] is the state after token t - 1
    hs = np.zeros((L + 1, bt, D, N))
    hs[0] = 0.0 if h0 is None else np.asarray(h0, dtype=np.float64)
    a_all = np.zeros((L, bt, D, N))
    for t in range(L):
        a_all[t] = np.exp(delta[:, :, t, None] * A[None, :, :])
        hs[t + 1] = a_all[t] * hs[t] + B[:, None, :, t] * delta[:, :, t, None] * x[:, :, t, None]
    g = np.zeros((bt, D, N)) if dhT is None else np.array(dhT, dtype=np.float64, copy=True)
    dx = np.zeros((bt, D, L))
    ddelta = np.zeros((bt, D, L))
    dA = np.zeros((D, N))
    dB = np.zeros((bt, N, L))
    dC = np.zeros((bt, N, L))
    for t in range(L - 1, -1, -1):
        dC[:, :, t] = np.einsum("bd,bdn->bn", dy[:, :, t], hs[t + 1])
        g = g + C[:, None, :, t] * dy[:, :, t, None]          # dL/dh_t, complete
        a, hp = a_all[t], hs[t]
        dlt, xt, Bt = delta[:, :, t, None], x[:, :, t, None], B[:, None, :, t]
        dx[:, :, t] = np.sum(g * Bt * dlt, axis=2)
        ddelta[:, :, t] = np.sum(g * (A[None] * a * hp + Bt * xt), axis=2)
        dA += np.sum(g * dlt * a * hp, axis=0)
        dB[:, :, t] = np.sum(g * dlt * xt, axis=1)
        g = a * g                                             # dL/dh_{t-1}, from step t
    return {"dx": dx, "ddelta": ddelta, "dA": dA, "dB": dB, "dC": dC, "dh0": g}
