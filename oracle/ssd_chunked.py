"""Chunk-wise fp64 evaluation of the Mamba-2 SSD forward pass.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Written from the NVIDIA developer blog "Accelerating Mamba-2 with
high-performance forward-pass kernels in NVIDIA CUDA Tile", section
"Mamba-2 architecture" (the jump formula of Fig. 1, the block output of
Figs. 2-3, and the decayed versions that follow), independently of
``ssd_seq.py``. Natural ``exp`` throughout; the base-2 rescaling of the
page's kernel 1 is an implementation device, not part of the result.

Within one chunk of ``Q`` tokens, with ``a_t = A * dt_t``:

  G       = inclusive cumulative sum of a over the chunk (chunk-local, the
            "Kernel 1" section: the sum restarts at every chunk)
  L[i, j] = exp(G_i - G_j) for i >= j, 0 above the diagonal (the causal
            mask M; exponents above the diagonal are set to -inf *before*
            exp, so no overflow can occur)
  Y       = exp(G)[:, None] * (C h^T) + (L o (C B^T)) (dt o X) + D X
  S       = X^T (exp(G_last - G) * dt o B)           (the chunk's own state)
  h_next  = exp(G_last) * h + S

with ``h`` the state entering the chunk (the chunk "checkpoint"), stored as
``[headdim, dstate]``. ``G_last`` is G at the chunk's last token.

Readings taken (each is listed with its reason in the design notes):

* The page's state jump writes ``(exp(G_last - G) o B) X^T``, which does not
  conform; the earlier undecayed jump ``B^T X`` fixes the orientation, so the
  decayed term is ``(exp(G_last - G) o B)^T X`` (here transposed once more
  into the headdim-major layout).
* ``dt`` multiplies the key: ``b_t = dt_t * B_t``; in ``Y`` the same factor
  is applied to X's rows, which is the same product.
* ``seqlen`` not a multiple of ``chunk``: the tail chunk is padded with
  tokens whose x, dt, B and C are zero (the kernel listings load with zero
  padding), so padded tokens neither decay nor feed the state.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .ssd_seq import heads_to_groups


def ssd_chunked(x, dt, A, B, C, D, chunk: int, init_state=None,
                heads: Optional[Sequence[int]] = None,
                return_intermediates: bool = False):
    """Evaluate the layer chunk by chunk, in float64.

    Same arguments and returns as ``ssd_sequential`` plus ``chunk``. With
    ``return_intermediates=True`` a third value is returned: a dict with
      ``G``      [batch, h, nchunks*chunk]   natural-log chunk-local cumsum
      ``states`` [batch, h, nchunks, headdim, dstate]   S of every chunk
      ``hprev``  [batch, h, nchunks, headdim, dstate]   state entering each chunk
    """
    if chunk <= 0:
        raise ValueError("chunk must be positive")
    x = np.asarray(x)
    bt, T, H, P = x.shape
    G_, N = np.asarray(B).shape[2], np.asarray(B).shape[3]
    heads = np.arange(H) if heads is None else np.asarray(heads, dtype=np.int64)
    nh = len(heads)
    grp = heads_to_groups(H, G_)[heads]
    nc = -(-T // chunk)
    Tp = nc * chunk

    As = np.asarray(A, dtype=np.float64)[heads]
    Ds = np.asarray(D, dtype=np.float64)[heads]
    causal = np.tril(np.ones((chunk, chunk), dtype=bool))

    y = np.zeros((bt, T, nh, P))
    final = np.zeros((bt, nh, P, N))
    if return_intermediates:
        G_all = np.zeros((bt, nh, Tp))
        S_all = np.zeros((bt, nh, nc, P, N))
        Hp_all = np.zeros((bt, nh, nc, P, N))

    for b in range(bt):
        if init_state is None:
            h = np.zeros((nh, P, N))
        else:
            h = np.array(np.asarray(init_state, dtype=np.float64)[b, heads], copy=True)
        for k in range(nc):
            lo, hi = k * chunk, min((k + 1) * chunk, T)
            n_real = hi - lo
            # chunk tensors, zero padded to `chunk` tokens, head-major
            Xk = np.zeros((nh, chunk, P))
            Xk[:, :n_real] = np.asarray(x[b, lo:hi], dtype=np.float64)[:, heads, :].transpose(1, 0, 2)
            dtk = np.zeros((nh, chunk))
            dtk[:, :n_real] = np.asarray(dt[b, lo:hi], dtype=np.float64)[:, heads].T
            Bk = np.zeros((nh, chunk, N))
            Bk[:, :n_real] = np.asarray(B[b, lo:hi], dtype=np.float64)[:, grp, :].transpose(1, 0, 2)
            Ck = np.zeros((nh, chunk, N))
            Ck[:, :n_real] = np.asarray(C[b, lo:hi], dtype=np.float64)[:, grp, :].transpose(1, 0, 2)

            Gk = np.cumsum(As[:, None] * dtk, axis=1)              # [nh, Q]
            Glast = Gk[:, -1]                                       # [nh]

            expo = Gk[:, :, None] - Gk[:, None, :]                  # G_i - G_j
            expo = np.where(causal[None], expo, -np.inf)
            Lk = np.exp(expo)                                       # decay o mask
            CB = np.matmul(Ck, Bk.transpose(0, 2, 1))               # [nh, Q, Q]
            dX = dtk[:, :, None] * Xk                                # dt o X
            Yk = (np.exp(Gk)[:, :, None] * np.matmul(Ck, h.transpose(0, 2, 1))
                  + np.matmul(Lk * CB, dX)
                  + Ds[:, None, None] * Xk)                          # [nh, Q, P]
            y[b, lo:hi] = Yk[:, :n_real].transpose(1, 0, 2)

            w = np.exp(Glast[:, None] - Gk) * dtk                    # [nh, Q]
            Sk = np.matmul(Xk.transpose(0, 2, 1), w[:, :, None] * Bk)   # [nh, P, N]
            if return_intermediates:
                G_all[b, :, k * chunk:(k + 1) * chunk] = Gk
                S_all[b, :, k] = Sk
                Hp_all[b, :, k] = h
            h = np.exp(Glast)[:, None, None] * h + Sk
        final[b] = h

    if return_intermediates:
        return y, final, {"G": G_all, "states": S_all, "hprev": Hp_all}
    return y, final
