"""Token-by-token fp64 evaluation of the Mamba-2 SSD recurrence.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Definition followed (NVIDIA developer blog, "Accelerating Mamba-2 with
high-performance forward-pass kernels in NVIDIA CUDA Tile", section
"Mamba-2 architecture", the core recurrence and the bullet list under it):

    h_t = exp(A * dt_t) * h_{t-1} + dt_t * B_t x_t^T
    y_t = c_t^T h_t + D * x_t

per head, where ``dt_t`` is one scalar per (token, head), ``x_t`` is the
head's value vector (headdim entries), ``B_t`` the key-like and ``c_t`` the
query-like vectors (dstate entries each, shared by every head of a group) and
``A``, ``D`` are per-head scalars.

Readings of the page taken here:

* ``y_t`` reads the *updated* state ``h_t`` (the first display of the
  section). The later shorthand display writes ``h_{t-1}``; the expanded
  output formula of the same section sums ``b`` up to and including the
  current token, and the causal mask keeps the diagonal, so ``h_t`` it is.
* The state is stored headdim-major: ``h[p, n]`` with ``p`` < headdim and
  ``n`` < dstate, i.e. the transpose of the page's (S, H) matrix; the update
  is ``h[p, n] += dt * x[p] * B[n]`` and ``y[p] = sum_n C[n] * h[p, n]``.
* Heads map to groups in contiguous blocks, ``group = head // (nheads //
  ngroups)`` (kernel 2 listing, the ``num_heads_per_group`` division).
* ``init_state=None`` means a zero initial state.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def heads_to_groups(nheads: int, ngroups: int) -> np.ndarray:
    """Group index of every head: contiguous blocks of nheads/ngroups heads."""
    if ngroups <= 0 or nheads % ngroups:
        raise ValueError("nheads must be a positive multiple of ngroups")
    return np.arange(nheads) // (nheads // ngroups)


def ssd_sequential(x, dt, A, B, C, D, init_state=None,
                   heads: Optional[Sequence[int]] = None):
    """Run the recurrence one token at a time, in float64.

    Args:
      x:  [batch, seqlen, nheads, headdim]
      dt: [batch, seqlen, nheads]
      A, D: [nheads]
      B, C: [batch, seqlen, ngroups, dstate]
      init_state: [batch, nheads, headdim, dstate] or None (zeros)
      heads: optional subset of head indices to evaluate (default: all)

    Returns ``(y, final_state)`` in float64: y ``[batch, seqlen, len(heads),
    headdim]`` and final_state ``[batch, len(heads), headdim, dstate]``.
    """
    x = np.asarray(x)
    bt, T, H, P = x.shape
    G, N = np.asarray(B).shape[2], np.asarray(B).shape[3]
    heads = np.arange(H) if heads is None else np.asarray(heads, dtype=np.int64)
    grp = heads_to_groups(H, G)[heads]

    xs = np.asarray(x, dtype=np.float64)[:, :, heads, :]          # [bt, T, h, P]
    dts = np.asarray(dt, dtype=np.float64)[:, :, heads]           # [bt, T, h]
    As = np.asarray(A, dtype=np.float64)[heads]                    # [h]
    Ds = np.asarray(D, dtype=np.float64)[heads]
    Bs = np.asarray(B, dtype=np.float64)[:, :, grp, :]             # [bt, T, h, N]
    Cs = np.asarray(C, dtype=np.float64)[:, :, grp, :]

    if init_state is None:
        h = np.zeros((bt, len(heads), P, N))
    else:
        h = np.array(np.asarray(init_state, dtype=np.float64)[:, heads], copy=True)

    y = np.empty((bt, T, len(heads), P))
    for t in range(T):
        step = dts[:, t]                                    # [bt, h]
        decay = np.exp(As[None, :] * step)                  # exp(A dt_t)
        b_t = step[:, :, None] * Bs[:, t]                   # dt_t B_t      [bt, h, N]
        h = decay[:, :, None, None] * h + xs[:, t, :, :, None] * b_t[:, :, None, :]
        y[:, t] = np.einsum("bhpn,bhn->bhp", h, Cs[:, t]) + Ds[None, :, None] * xs[:, t]
    return y, h
