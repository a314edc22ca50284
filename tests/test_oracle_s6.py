"""Pins for the S6 (Mamba-1 selective scan) oracle, CPU only.

* s1 -- the page's printed discretization values: with delta = 0.5 and
  alpha = 0.9, A = log(alpha) / delta and B = -log(alpha) give a_ = 0.9000
  and b_ = 0.0527 ("Mamba: The Hard Way", Part 5); the scan then is the
  exponential moving average y_t = sum_s 0.9^(t - s) * 0.0527 * x_s
  (golden file tests/golden/ema_discretize.json).
* s2 -- reduction to the Mamba-2 SSD recurrence (pinned separately): when
  A[d, n] does not depend on n, channel d is an SSD head with headdim 1,
  dt = delta[d], A_h = A[d, 0], the shared B and C as one group and D = 0.
* s3 -- delta = 0 holds the state: y_t = C_t . h0.
* s4 -- chaining: a scan of T tokens equals a scan of T1 tokens followed by
  one of T - T1 tokens from its final state.
* s5 -- brute force on a tiny input: the unrolled sum
  h_t = sum_s (prod_{s < r <= t} a_r) b_s x_s (+ prod a h0).
Planted mutants in a copy of the oracle must each fail one of s1-s5.
"""
import os
import types

import numpy as np
import pytest

from oracle import ssd_sequential
from oracle.s6 import s6_sequential

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden", "ema_discretize.json")


def _inputs(seed, bt=2, D=3, N=4, L=9, with_h0=True):
    r = np.random.default_rng(seed)
    x = r.standard_normal((bt, D, L))
    delta = np.log1p(np.exp(r.standard_normal((bt, D, L)) - 1.0))
    A = -np.exp(r.uniform(-1.0, 1.0, (D, N)))
    B = r.standard_normal((bt, N, L))
    C = r.standard_normal((bt, N, L))
    h0 = r.standard_normal((bt, D, N)) if with_h0 else None
    return x, delta, A, B, C, h0


def _golden():
    import json
    with open(GOLDEN) as f:
        g = json.load(f)
    return {"alpha": g["inputs"]["alpha"], "delta": g["inputs"]["delta"], "a_": g["printed"]["a_bar"],
            "b_": g["printed"]["b_bar"]}


def pin_page_discretization(scan):
    g = _golden()
    alpha, dlt = g["alpha"], g["delta"]
    L = 12
    x = np.random.default_rng(0).standard_normal((1, 1, L))
    A = np.array([[np.log(alpha) / dlt]])
    B = np.full((1, 1, L), -np.log(alpha))
    C = np.ones((1, 1, L))
    y, _ = scan(x, np.full((1, 1, L), dlt), A, B, C, None)
    a_, b_ = np.exp(dlt * A[0, 0]), B[0, 0, 0] * dlt
    if abs(a_ - g["a_"]) > 5e-5 or abs(b_ - g["b_"]) > 5e-5:
        return "discretization differs from the printed values"
    want = np.array([sum(a_ ** (t - s) * b_ * x[0, 0, s] for s in range(t + 1)) for t in range(L)])
    if not np.allclose(y[0, 0], want, rtol=1e-12, atol=1e-12):
        return "not the moving average"
    return None


def pin_reduces_to_ssd(scan):
    x, delta, A, B, C, h0 = _inputs(1)
    A = np.repeat(A[:, :1], A.shape[1], axis=1)            # A[d, n] = A[d, 0]
    y, hT = scan(x, delta, A, B, C, h0)
    # SSD layout: x [bt, T, H, P=1], dt [bt, T, H], B/C [bt, T, G=1, N]
    ys, fs = ssd_sequential(x.transpose(0, 2, 1)[..., None], delta.transpose(0, 2, 1), A[:, 0],
                            B.transpose(0, 2, 1)[:, :, None, :], C.transpose(0, 2, 1)[:, :, None, :],
                            np.zeros(x.shape[1]), h0[:, :, None, :])
    if not np.allclose(y, ys[..., 0].transpose(0, 2, 1), rtol=1e-12, atol=1e-12):
        return "y differs from the SSD recurrence with headdim 1"
    if not np.allclose(hT, fs[:, :, 0, :], rtol=1e-12, atol=1e-12):
        return "final state differs from the SSD recurrence"
    return None


def pin_zero_delta_holds(scan):
    x, delta, A, B, C, h0 = _inputs(2)
    y, hT = scan(x, np.zeros_like(delta), A, B, C, h0)
    want = np.einsum("bdn,bnt->bdt", h0, C)
    if not (np.allclose(y, want, rtol=1e-12, atol=1e-12) and np.allclose(hT, h0, rtol=0, atol=0)):
        return "delta = 0 does not hold the state"
    return None


def pin_chaining(scan):
    x, delta, A, B, C, h0 = _inputs(3, L=11)
    y, hT = scan(x, delta, A, B, C, h0)
    y1, h1 = scan(x[..., :4], delta[..., :4], A, B[..., :4], C[..., :4], h0)
    y2, h2 = scan(x[..., 4:], delta[..., 4:], A, B[..., 4:], C[..., 4:], h1)
    if not (np.allclose(y, np.concatenate([y1, y2], -1), rtol=1e-12, atol=1e-12)
            and np.allclose(hT, h2, rtol=1e-12, atol=1e-12)):
        return "chained scans differ from one scan"
    return None


def pin_brute_force(scan):
    x, delta, A, B, C, h0 = _inputs(4, bt=1, D=2, N=3, L=6)
    y, hT = scan(x, delta, A, B, C, h0)
    bt, D, L = x.shape
    N = A.shape[1]
    for d in range(D):
        for t in range(L):
            acc = 0.0
            for n in range(N):
                a = [np.exp(delta[0, d, r] * A[d, n]) for r in range(L)]
                h = np.prod(a[:t + 1]) * h0[0, d, n]
                h += sum(np.prod(a[s + 1:t + 1]) * B[0, n, s] * delta[0, d, s] * x[0, d, s] for s in range(t + 1))
                acc += C[0, n, t] * h
            if abs(acc - y[0, d, t]) > 1e-10 * max(1.0, abs(acc)):
                return f"brute force differs at d={d}, t={t}"
    return None


S6_PINS = [pin_page_discretization, pin_reduces_to_ssd, pin_zero_delta_holds, pin_chaining, pin_brute_force]


@pytest.mark.parametrize("pin", S6_PINS, ids=lambda f: f.__name__)
def test_s6_oracle_pins(pin):
    assert pin(s6_sequential) is None


S6_MUTANTS = {
    "b_without_delta": ("b_ = B[:, None, :, t] * delta[:, :, t, None]", "b_ = B[:, None, :, t] + 0 * delta[:, :, t, None]"),
    "decay_sign": ("a_ = np.exp(delta[:, :, t, None] * A[None, :, :])", "a_ = np.exp(-delta[:, :, t, None] * A[None, :, :])"),
    "y_reads_old_state": ("        h = a_ * h + b_ * x[:, :, t, None]\n        y[:, :, t] = np.einsum(\"bdn,bn->bd\", h, C[:, :, t])",
                          "        y[:, :, t] = np.einsum(\"bdn,bn->bd\", h, C[:, :, t])\n        h = a_ * h + b_ * x[:, :, t, None]"),
    "y_contracts_B": ('y[:, :, t] = np.einsum("bdn,bn->bd", h, C[:, :, t])', 'y[:, :, t] = np.einsum("bdn,bn->bd", h, B[:, :, t])'),
    "A_transposed": ("a_ = np.exp(delta[:, :, t, None] * A[None, :, :])", "a_ = np.exp(delta[:, :, t, None] * A.T[None, :, :])"),
    "h0_ignored": ("h = np.zeros((bt, D, N)) if h0 is None else np.array(h0, dtype=np.float64, copy=True)",
                   "h = np.zeros((bt, D, N))"),
}


@pytest.mark.parametrize("name", sorted(S6_MUTANTS))
def test_s6_mutant_caught(name):
    old, new = S6_MUTANTS[name]
    with open(os.path.join(ROOT, "oracle", "s6.py")) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("mutant_s6")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    caught = False
    for pin in S6_PINS:
        try:
            if pin(mod.s6_sequential) is not None:
                caught = True
                break
        except (ValueError, IndexError, FloatingPointError):
            caught = True
            break
    assert caught, f"no pin rejects the mutant {name}"
