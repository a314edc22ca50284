"""Pins for the fp64 oracle: checks against facts fixed outside the oracle.

Every check takes a forward callable
``fwd(x, dt, A, B, C, D, init_state) -> (y, final_state)`` so the same pins
run on the sequential oracle, on the chunked oracle at several chunk sizes,
and on deliberately broken copies of either (``test_oracle_mutations.py``).

None of these checks re-types the oracle's own formula. Each one uses a
different route to the same result:

  p1  dt == 0 keeps the state: final == init bit for bit, and y = D x when
      the initial state is zero (CUDA Tile blog, "Mamba-2 architecture",
      the remark that dt = 0 leaves the state unchanged).
  p2  A == 0 removes the decay: the layer is causal linear attention, one
      dense T x T masked product per head (same section, the undecayed
      block formula Y = C h + ((C B^T) . M) X + D X and the remark that
      without decay Mamba-2 is linear attention).
  p5  brute force on tiny inputs: the fully unrolled sum of the decayed
      recurrence, every term an explicit product of exponentials, summed
      with math.fsum (same section, the unrolled h_{t+T} display).
  p6  the worked discretisation example printed in "Mamba: The Hard Way"
      Part 5, plus the Part 2 exponential-moving-average definition it
      rebuilds (tests/golden/ema_discretize.json).
  p7  chaining: a call over the whole sequence equals a call over a prefix
      followed by a call over the rest that starts from the prefix's final
      state (CUDA Tile blog, kernel 2: the final state is fed back as the
      next call's initial state).
  p8  group broadcast: heads of one group see that group's B and C only
      (kernel 2 listing, head // num_heads_per_group).
  p9  superposition: at fixed dt, A, B, C, D the layer is linear in
      (x, initial state) jointly (the recurrence is linear in h and x).
  p10 one token: y = C.(exp(A dt) h0 + dt x B^T) + D x in closed form.
  p11 constant per-token decay alpha: the decay between tokens i >= j is
      alpha**(i - j), evaluated with integer powers instead of a cumulative
      sum (the "Mamba-2 architecture" remark that exp(G - G^T) holds
      exp(g_i - g_j)).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def rand_layer(seed, bt=2, T=12, H=4, P=3, N=5, G=2, init=True, dt_zero_frac=0.0):
    """Small random layer with the page's sign conventions (A < 0, dt >= 0)."""
    r = _rng(seed)
    x = r.standard_normal((bt, T, H, P))
    B = r.standard_normal((bt, T, G, N))
    C = r.standard_normal((bt, T, G, N))
    dt = np.logaddexp(0.0, r.standard_normal((bt, T, H)) - 1.0)
    if dt_zero_frac:
        dt[r.random(dt.shape) < dt_zero_frac] = 0.0
    A = -np.exp(r.uniform(np.log(0.5), np.log(4.0), H))
    D = r.standard_normal(H)
    h0 = r.standard_normal((bt, H, P, N)) if init else None
    return x, dt, A, B, C, D, h0


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


def assert_close(a, b, tol=1e-12, what=""):
    e = rel_err(a, b)
    assert e <= tol, f"{what}: relative error {e:.3e} > {tol:.1e}"


# ---------------------------------------------------------------- p1
def pin_dt_zero(fwd):
    x, dt, A, B, C, D, h0 = rand_layer(11, T=9)
    dt = np.zeros_like(dt)
    y, fin = fwd(x, dt, A, B, C, D, h0)
    assert np.array_equal(np.asarray(fin), h0), "dt == 0 must leave the state unchanged bit for bit"
    # with a zero initial state only the skip term survives, exactly
    y0, fin0 = fwd(x, dt, A, B, C, D, None)
    assert np.array_equal(np.asarray(fin0), np.zeros_like(h0))
    assert np.array_equal(np.asarray(y0), D[None, None, :, None] * x), "dt == 0, h0 == 0 must give y = D x"
    # with a nonzero initial state y_t = C_t . h0 + D x_t, summed over dstate
    H, G = x.shape[2], B.shape[2]
    g = np.arange(H) // (H // G)
    expect = np.zeros_like(x)
    for b in range(x.shape[0]):
        for t in range(x.shape[1]):
            for h in range(H):
                for p in range(x.shape[3]):
                    expect[b, t, h, p] = math.fsum(C[b, t, g[h], n] * h0[b, h, p, n]
                                                   for n in range(B.shape[3])) + D[h] * x[b, t, h, p]
    assert_close(y, expect, 1e-13, "p1 held state read by C")


# ---------------------------------------------------------------- p2
def pin_linear_attention(fwd):
    x, dt, A, B, C, D, h0 = rand_layer(12, T=17, P=3, N=5)
    A = np.zeros_like(A)
    y, fin = fwd(x, dt, A, B, C, D, h0)
    bt, T, H, P = x.shape
    g = np.arange(H) // (H // B.shape[2])
    mask = np.tril(np.ones((T, T)))
    ey = np.empty_like(x)
    efin = np.empty_like(h0)
    for b in range(bt):
        for h in range(H):
            Cg, Bg, X = C[b, :, g[h]], B[b, :, g[h]], x[b, :, h]
            scores = (Cg @ Bg.T) * mask                      # causal, diagonal kept
            ey[b, :, h] = Cg @ h0[b, h].T + scores @ (dt[b, :, h][:, None] * X) + D[h] * X
            efin[b, h] = h0[b, h] + X.T @ (dt[b, :, h][:, None] * Bg)
    assert_close(y, ey, 1e-12, "p2 linear attention y")
    assert_close(fin, efin, 1e-12, "p2 linear attention final state")


# ---------------------------------------------------------------- p5
def _unrolled(x, dt, A, B, C, D, h0, g):
    """h_t = exp(sum_{s<=t} a_s) h0 + sum_{j<=t} exp(sum_{j<s<=t} a_s) dt_j x_j B_j^T."""
    bt, T, H, P = x.shape
    N = B.shape[3]
    y = np.zeros_like(x)
    fin = np.zeros((bt, H, P, N))
    for b in range(bt):
        for h in range(H):
            a = [A[h] * dt[b, s, h] for s in range(T)]
            for t in range(T):
                for p in range(P):
                    hs = []
                    for n in range(N):
                        terms = [math.exp(math.fsum(a[: t + 1])) * (h0[b, h, p, n] if h0 is not None else 0.0)]
                        for j in range(t + 1):
                            terms.append(math.exp(math.fsum(a[j + 1: t + 1])) * dt[b, j, h]
                                         * x[b, j, h, p] * B[b, j, g[h], n])
                        hs.append(math.fsum(terms))
                    y[b, t, h, p] = math.fsum(C[b, t, g[h], n] * hs[n] for n in range(N)) + D[h] * x[b, t, h, p]
                    if t == T - 1:
                        fin[b, h, p, :] = hs
    return y, fin


def pin_bruteforce(fwd):
    for seed, (T, P, N, G, H) in enumerate([(8, 2, 2, 1, 2), (7, 2, 3, 2, 2), (5, 3, 2, 1, 1)]):
        x, dt, A, B, C, D, h0 = rand_layer(100 + seed, bt=1, T=T, H=H, P=P, N=N, G=G)
        g = np.arange(H) // (H // G)
        ey, efin = _unrolled(x, dt, A, B, C, D, h0, g)
        y, fin = fwd(x, dt, A, B, C, D, h0)
        assert_close(y, ey, 1e-12, f"p5 unrolled y (case {seed})")
        assert_close(fin, efin, 1e-12, f"p5 unrolled final (case {seed})")


# ---------------------------------------------------------------- p6
def pin_ema_worked_example(fwd):
    with open(os.path.join(GOLDEN, "ema_discretize.json")) as f:
        gold = json.load(f)
    alpha = gold["inputs"]["alpha"]
    delta = gold["inputs"]["delta"]
    half_ulp = 0.5 * 10.0 ** (-gold["printed_decimals"])
    # a = log(alpha)/delta is the (negative) A, delta is dt, b = -log(alpha) is B.
    A = np.array([math.log(alpha) / delta])
    Bv = -math.log(alpha)
    one = np.ones((1, 1, 1, 1))
    dt = np.full((1, 1, 1), delta)
    # a single token with x = 0 from h0 = 1 reads back exp(A dt) = a_bar
    y, _ = fwd(np.zeros((1, 1, 1, 1)), dt, A, Bv * one, one, np.zeros(1), one)
    assert abs(float(y.ravel()[0]) - gold["printed"]["a_bar"]) <= half_ulp, "p6 a_bar"
    # a single token with x = 1 from h0 = 0 reads back dt * B = b_bar
    y, _ = fwd(one, dt, A, Bv * one, one, np.zeros(1), None)
    assert abs(float(y.ravel()[0]) - gold["printed"]["b_bar"]) <= half_ulp, "p6 b_bar"

    # the same discretisation over a sequence: closed-form geometric sum
    T = 40
    xs = _rng(6).standard_normal(T)
    y, fin = fwd(xs.reshape(1, T, 1, 1), np.full((1, T, 1), delta), A,
                 np.full((1, T, 1, 1), Bv), np.ones((1, T, 1, 1)), np.zeros(1), None)
    a_bar, b_bar = alpha, delta * Bv
    expect = [math.fsum(a_bar ** (t - s) * b_bar * xs[s] for s in range(t + 1)) for t in range(T)]
    assert_close(y.ravel(), expect, 1e-12, "p6 geometric sum")

    # Part 2's EMA, h = alpha h + (1 - alpha) x, is A = log(alpha), dt = 1, B = 1 - alpha
    h, ema = 0.0, []
    for k in range(T):
        h = alpha * h + (1 - alpha) * xs[k]
        ema.append(h)
    y, fin = fwd(xs.reshape(1, T, 1, 1), np.ones((1, T, 1)), np.array([math.log(alpha)]),
                 np.full((1, T, 1, 1), 1 - alpha), np.ones((1, T, 1, 1)), np.zeros(1), None)
    assert_close(y.ravel(), ema, 1e-12, "p6 EMA")
    assert abs(float(fin.ravel()[0]) - ema[-1]) <= 1e-12 * max(1.0, abs(ema[-1]))


# ---------------------------------------------------------------- p7
def pin_chaining(fwd, split_points=(4, 8, 13)):
    x, dt, A, B, C, D, h0 = rand_layer(17, T=24)
    y, fin = fwd(x, dt, A, B, C, D, h0)
    for s in split_points:
        y1, f1 = fwd(x[:, :s], dt[:, :s], A, B[:, :s], C[:, :s], D, h0)
        y2, f2 = fwd(x[:, s:], dt[:, s:], A, B[:, s:], C[:, s:], D, f1)
        assert_close(np.concatenate([y1, y2], axis=1), y, 1e-12, f"p7 chained y at {s}")
        assert_close(f2, fin, 1e-12, f"p7 chained final at {s}")


# ---------------------------------------------------------------- p8
def pin_group_broadcast(fwd):
    x, dt, A, B, C, D, h0 = rand_layer(18, T=10, H=6, G=3)
    y, fin = fwd(x, dt, A, B, C, D, h0)
    per = 2
    for grp in range(3):
        hs = slice(grp * per, (grp + 1) * per)
        ys, fs = fwd(x[:, :, hs], dt[:, :, hs], A[hs], B[:, :, grp:grp + 1], C[:, :, grp:grp + 1],
                     D[hs], h0[:, hs])
        assert_close(ys, y[:, :, hs], 1e-13, f"p8 group {grp} y")
        assert_close(fs, fin[:, hs], 1e-13, f"p8 group {grp} final")


# ---------------------------------------------------------------- p9
def pin_superposition(fwd):
    x, dt, A, B, C, D, h0 = rand_layer(19, T=11)
    x2, _, _, _, _, _, h02 = rand_layer(20, T=11)
    ya, fa = fwd(x, dt, A, B, C, D, h0)
    yb, fb = fwd(x2, dt, A, B, C, D, h02)
    yc, fc = fwd(2.0 * x - 3.0 * x2, dt, A, B, C, D, 2.0 * h0 - 3.0 * h02)
    assert_close(yc, 2.0 * ya - 3.0 * yb, 1e-12, "p9 y")
    assert_close(fc, 2.0 * fa - 3.0 * fb, 1e-12, "p9 final")


# ---------------------------------------------------------------- p10
def pin_single_token(fwd):
    x, dt, A, B, C, D, h0 = rand_layer(21, T=1, P=3, N=4)
    y, fin = fwd(x, dt, A, B, C, D, h0)
    H = x.shape[2]
    g = np.arange(H) // (H // B.shape[2])
    for b in range(x.shape[0]):
        for h in range(H):
            hn = math.exp(A[h] * dt[b, 0, h]) * h0[b, h] + dt[b, 0, h] * np.outer(x[b, 0, h], B[b, 0, g[h]])
            assert_close(fin[b, h], hn, 1e-13, "p10 state")
            assert_close(y[b, 0, h], hn @ C[b, 0, g[h]] + D[h] * x[b, 0, h], 1e-13, "p10 y")


# ---------------------------------------------------------------- p11
def pin_constant_decay(fwd):
    x, dt, A, B, C, D, h0 = rand_layer(22, T=20, P=3, N=4)
    bt, T, H, P = x.shape
    dt = np.full_like(dt, 0.37)
    y, fin = fwd(x, dt, A, B, C, D, h0)
    g = np.arange(H) // (H // B.shape[2])
    i = np.arange(T)
    for b in range(bt):
        for h in range(H):
            alpha = math.exp(A[h] * 0.37)
            powers = np.where(i[:, None] >= i[None, :],
                              alpha ** np.maximum(i[:, None] - i[None, :], 0), 0.0)   # Toeplitz alpha^(i-j)
            Cg, Bg, X = C[b, :, g[h]], B[b, :, g[h]], x[b, :, h]
            carried = (alpha ** (i + 1))[:, None] * (Cg @ h0[b, h].T)
            ey = carried + ((Cg @ Bg.T) * powers) @ (0.37 * X) + D[h] * X
            assert_close(y[:, :, h][b], ey, 1e-12, "p11 y")
            efin = alpha ** T * h0[b, h] + X.T @ ((0.37 * alpha ** (T - 1 - i))[:, None] * Bg)
            assert_close(fin[b, h], efin, 1e-12, "p11 final")


ALL_PINS = {
    "p1_dt_zero": pin_dt_zero,
    "p2_linear_attention": pin_linear_attention,
    "p5_bruteforce": pin_bruteforce,
    "p6_ema_worked_example": pin_ema_worked_example,
    "p7_chaining": pin_chaining,
    "p8_group_broadcast": pin_group_broadcast,
    "p9_superposition": pin_superposition,
    "p10_single_token": pin_single_token,
    "p11_constant_decay": pin_constant_decay,
}
