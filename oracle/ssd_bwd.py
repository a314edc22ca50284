"""fp64 gradients of the Mamba-2 SSD layer (the backward pass).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The layer is the forward recurrence of ``ssd_seq.py`` (NVIDIA developer
blog, "Accelerating Mamba-2 with high-performance forward-pass kernels in
NVIDIA CUDA Tile", section "Mamba-2 architecture"):

    h_t = exp(A dt_t) h_{t-1} + dt_t x_t B_t^T      (state held [p, n])
    y_t = h_t C_t + D x_t

with ``final = h_{T-1}``. For a loss with upstream gradients ``dy`` (same
shape as y) and ``dfinal`` (same shape as the final state, zeros when None)
the functions here return every input's gradient: dx, ddt, dA, dB, dC, dD and
dinit (the initial state's).

Two evaluations, written independently of each other:

* ``ssd_bwd_sequential`` -- reverse mode through the token recurrence. As the
  "Part 3" derivation of Sasha Rush's "Mamba: The Hard Way" shows for the
  scalar scan, the adjoint of the state obeys the same recurrence run
  backwards in time, dh_{t-1} = alpha_t dh_t (+ the output's C_t dy_t), and
  the gradients of the per-step coefficients need both the forward states and
  these backward ones.
* ``ssd_bwd_chunked`` -- the same gradients from the chunked "jump" form of
  the forward pass (``ssd_chunked.py``), differentiated block by block: the
  intra-chunk products C B^T and dy x^T under the decay mask, the carried
  state entering each chunk, and a reverse pass of the state adjoint over the
  chunk boundaries. Natural ``exp``, no base-2 rescaling.

Both upcast every input to float64. Group sums: B and C are shared by the
heads of a group, so dB and dC add the contributions of all of them.
"""
from __future__ import annotations

import numpy as np

from .ssd_seq import heads_to_groups


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _zeros_like_grads(bt, T, H, P, N, G):
    return {
        "dx": np.zeros((bt, T, H, P)),
        "ddt": np.zeros((bt, T, H)),
        "dA": np.zeros(H),
        "dB": np.zeros((bt, T, G, N)),
        "dC": np.zeros((bt, T, G, N)),
        "dD": np.zeros(H),
        "dinit": np.zeros((bt, H, P, N)),
    }


def ssd_bwd_sequential(x, dt, A, B, C, D, dy, init_state=None, dfinal=None):
    """Gradients by reverse mode through the token-by-token recurrence.

    Shapes as ``ssd_sequential``; ``dy`` like y ``[batch, seqlen, nheads,
    headdim]``, ``dfinal`` like the final state ``[batch, nheads, headdim,
    dstate]`` or None. Returns a dict of float64 arrays named after the
    inputs (dx, ddt, dA, dB, dC, dD, dinit).
    """
    x, dt, A, B, C, D, dy = map(_f64, (x, dt, A, B, C, D, dy))
    bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    grp = heads_to_groups(H, G)
    out = _zeros_like_grads(bt, T, H, P, N, G)
    for b in range(bt):
        for h in range(H):
            g = grp[h]
            a = A[h]
            # forward: states[t + 1] is h_t, states[0] the initial state
            states = np.zeros((T + 1, P, N))
            if init_state is not None:
                states[0] = _f64(init_state)[b, h]
            alpha = np.exp(a * dt[b, :, h])
            for t in range(T):
                states[t + 1] = alpha[t] * states[t] + dt[b, t, h] * np.outer(x[b, t, h], B[b, t, g])
            # backward: dh is the adjoint of h_t, walked from the end
            dh = np.zeros((P, N)) if dfinal is None else _f64(dfinal)[b, h].copy()
            for t in range(T - 1, -1, -1):
                xt, Bt, Ct, dyt, dtt = x[b, t, h], B[b, t, g], C[b, t, g], dy[b, t, h], dt[b, t, h]
                # y_t = h_t C_t + D x_t
                dh = dh + np.outer(dyt, Ct)
                out["dC"][b, t, g] += dyt @ states[t + 1]
                out["dD"][h] += dyt @ xt
                # h_t = alpha_t h_{t-1} + dt_t x_t B_t^T, alpha_t = exp(A dt_t)
                out["dx"][b, t, h] += D[h] * dyt + dtt * (dh @ Bt)
                out["dB"][b, t, g] += dtt * (xt @ dh)
                dalpha = np.sum(dh * states[t])
                out["ddt"][b, t, h] += xt @ dh @ Bt + dalpha * alpha[t] * a
                out["dA"][h] += dalpha * alpha[t] * dtt
                dh = alpha[t] * dh
            out["dinit"][b, h] = dh
    return out


def ssd_bwd_chunked(x, dt, A, B, C, D, dy, chunk: int, init_state=None, dfinal=None):
    """Gradients from the chunked form, chunk length ``chunk`` (a ragged last
    chunk is zero padded: its padded tokens have dt = 0 and contribute
    nothing). Same arguments and result as ``ssd_bwd_sequential``.

    Per chunk, with G the chunk-local inclusive cumsum of A dt, E = exp(G),
    L_ij = exp(G_i - G_j) for i >= j (else 0), w_j = exp(G_last - G_j) dt_j,
    Hprev the state entering the chunk and dHn the adjoint of the state
    leaving it:

      dx   = (L o CB o dt_j)^T dY + diag(w) B dHn^T + D dY
      dB_h = (L o DX o dt_j)^T C  + diag(w) X dHn
      dC_h = (L o DX o dt_j) B    + diag(E) dY Hprev
      dHprev = exp(G_last) dHn + dY^T diag(E) C

    with CB = C B^T and DX = dY X^T. The gradient with respect to G collects
    the row and column sums of Z = L o CB o DX o dt_j (+ rows, - columns),
    E_i dy_i . (Hprev C_i), -w_j x_j . (dHn B_j), and at the last token
    exp(G_last) <dHn, Hprev> + sum_j w_j x_j . (dHn B_j); it reaches dt and A
    through G_i = A sum_{s <= i} dt_s.
    """
    if chunk <= 0:
        raise ValueError("chunk must be positive")
    x, dt, A, B, C, D, dy = map(_f64, (x, dt, A, B, C, D, dy))
    bt, T, H, P = x.shape
    G_, N = B.shape[2], B.shape[3]
    grp = heads_to_groups(H, G_)
    nc = -(-T // chunk)
    Q = chunk
    out = _zeros_like_grads(bt, T, H, P, N, G_)
    causal = np.tril(np.ones((Q, Q), dtype=bool))

    def tiles(b, h, k):
        lo, hi = k * Q, min((k + 1) * Q, T)
        n = hi - lo
        g = grp[h]
        Xk, dYk = np.zeros((Q, P)), np.zeros((Q, P))
        Bk, Ck = np.zeros((Q, N)), np.zeros((Q, N))
        dtk = np.zeros(Q)
        Xk[:n], dYk[:n] = x[b, lo:hi, h], dy[b, lo:hi, h]
        Bk[:n], Ck[:n] = B[b, lo:hi, g], C[b, lo:hi, g]
        dtk[:n] = dt[b, lo:hi, h]
        return lo, n, g, Xk, dYk, Bk, Ck, dtk

    for b in range(bt):
        for h in range(H):
            a = A[h]
            # forward over the chunks: the state entering each one
            Hprev = np.zeros((nc, P, N))
            hcur = np.zeros((P, N)) if init_state is None else _f64(init_state)[b, h].copy()
            for k in range(nc):
                _, _, _, Xk, _, Bk, _, dtk = tiles(b, h, k)
                Gk = np.cumsum(a * dtk)
                Hprev[k] = hcur
                w = np.exp(Gk[-1] - Gk) * dtk
                hcur = np.exp(Gk[-1]) * hcur + Xk.T @ (w[:, None] * Bk)
            # backward over the chunks, last first
            dHn = np.zeros((P, N)) if dfinal is None else _f64(dfinal)[b, h].copy()
            for k in range(nc - 1, -1, -1):
                lo, n, g, Xk, dYk, Bk, Ck, dtk = tiles(b, h, k)
                Gk = np.cumsum(a * dtk)
                Gl = Gk[-1]
                E = np.exp(Gk)
                w = np.exp(Gl - Gk) * dtk
                L = np.exp(np.where(causal, Gk[:, None] - Gk[None, :], -np.inf))
                CB = Ck @ Bk.T
                DX = dYk @ Xk.T
                W1 = L * CB * dtk[None, :]
                W2 = L * DX * dtk[None, :]
                dHnB = Bk @ dHn.T                       # [Q, P]: row j is dHn B_j
                HpC = Ck @ Hprev[k].T                   # [Q, P]: row i is Hprev C_i
                dx = W1.T @ dYk + w[:, None] * dHnB + D[h] * dYk
                dBh = W2.T @ Ck + w[:, None] * (Xk @ dHn)
                dCh = W2 @ Bk + E[:, None] * (dYk @ Hprev[k])
                Z = W1 * DX
                bvec = np.sum(Xk * dHnB, axis=1)
                avec = np.sum(dYk * HpC, axis=1)
                dG = E * avec + Z.sum(axis=1) - Z.sum(axis=0) - w * bvec
                dG[-1] += np.exp(Gl) * np.sum(dHn * Hprev[k]) + np.sum(w * bvec)
                ddt_direct = (L * CB * DX).sum(axis=0) + np.exp(Gl - Gk) * bvec
                ddt = ddt_direct + a * np.cumsum(dG[::-1])[::-1]
                out["dA"][h] += np.sum(dG * np.cumsum(dtk))
                out["dD"][h] += np.sum(dYk * Xk)
                out["dx"][b, lo:lo + n, h] = dx[:n]
                out["ddt"][b, lo:lo + n, h] = ddt[:n]
                out["dB"][b, lo:lo + n, g] += dBh[:n]
                out["dC"][b, lo:lo + n, g] += dCh[:n]
                dHn = np.exp(Gl) * dHn + dYk.T @ (E[:, None] * Ck)
            out["dinit"][b, h] = dHn
    return out
