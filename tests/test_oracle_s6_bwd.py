"""Pins for the S6 gradient oracle (``oracle.s6.s6_bwd_sequential``), CPU only.

* g1 -- central finite differences of the pinned forward oracle
  ``s6_sequential`` (tests/test_oracle_s6.py) for every element of every
  input, for the loss sum(y * dy) + sum(hT * dhT).
* g2 -- closed forms with delta = 0 (the state holds h0): dx = dB = dA = 0,
  dC_t = sum_d dy_t h0, dh0 = dhT + sum_t C_t dy_t, and
  ddelta_t = sum_n g_t (A h0 + B_t x_t) with g_t = dhT + sum_{s >= t} C_s dy_s.
* g3 -- linearity in (dy, dhT).
* g4 -- reduction to the SSD gradient oracle (pinned separately in
  tests/test_oracle_bwd.py): when A[d, n] does not depend on n, channel d is
  an SSD head with headdim 1, so dx, ddelta (ddt), dB, dC and dh0 (dinit)
  equal the SSD gradients and sum_n dA[d, n] equals the SSD's dA[d].
Planted mutants in a copy of the oracle must each fail one of g1-g4.
"""
import inspect
import types

import numpy as np
import pytest

import oracle.s6 as s6mod
from oracle import ssd_bwd_sequential
from oracle.s6 import s6_bwd_sequential, s6_sequential


def _inputs(seed, bt=2, D=3, N=2, L=6, with_h0=True):
    r = np.random.default_rng(seed)
    x = r.standard_normal((bt, D, L))
    delta = np.log1p(np.exp(r.standard_normal((bt, D, L)) - 1.0))
    A = -np.exp(r.uniform(-1.0, 1.0, (D, N)))
    B = r.standard_normal((bt, N, L))
    C = r.standard_normal((bt, N, L))
    h0 = r.standard_normal((bt, D, N)) if with_h0 else None
    dy = r.standard_normal((bt, D, L))
    dhT = r.standard_normal((bt, D, N))
    return x, delta, A, B, C, h0, dy, dhT


def _loss(args, dy, dhT):
    y, hT = s6_sequential(*args)
    return float(np.sum(y * dy) + np.sum(hT * dhT))


def pin_finite_differences(bwd, seed=3):
    x, delta, A, B, C, h0, dy, dhT = _inputs(seed)
    g = bwd(x, delta, A, B, C, dy, h0, dhT)
    args = [x, delta, A, B, C, h0]
    names = {0: "dx", 1: "ddelta", 2: "dA", 3: "dB", 4: "dC", 5: "dh0"}
    eps = 1e-6
    for i, name in names.items():
        base = args[i]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus = [a.copy() if j == i else a for j, a in enumerate(args)]
            minus = [a.copy() if j == i else a for j, a in enumerate(args)]
            plus[i][idx] += eps
            minus[i][idx] -= eps
            fd[idx] = (_loss(plus, dy, dhT) - _loss(minus, dy, dhT)) / (2 * eps)
        scale = max(float(np.max(np.abs(fd))), 1e-12)
        if float(np.max(np.abs(g[name] - fd))) > 1e-6 * scale:
            return f"{name} differs from finite differences"
    return None


def pin_closed_forms(bwd):
    x, delta, A, B, C, h0, dy, dhT = _inputs(4)
    delta = np.zeros_like(delta)
    g = bwd(x, delta, A, B, C, dy, h0, dhT)
    L = x.shape[2]
    for k in ("dx", "dB", "dA"):
        if np.max(np.abs(g[k])) > 1e-14:
            return f"{k} is not zero with delta = 0"
    if not np.allclose(g["dC"], np.einsum("bdt,bdn->bnt", dy, h0), rtol=1e-12, atol=1e-12):
        return "dC differs from sum_d dy h0"
    cdy = np.einsum("bnt,bdt->bdnt", C, dy)                    # C_t dy_t per (b, d, n, t)
    gt = dhT[..., None] + np.cumsum(cdy[..., ::-1], axis=-1)[..., ::-1]
    if not np.allclose(g["dh0"], gt[..., 0], rtol=1e-12, atol=1e-12):
        return "dh0 differs from dhT + sum_t C_t dy_t"
    want = np.einsum("bdnt,bdnt->bdt", gt, A[None, :, :, None] * h0[..., None] + B[:, None, :, :] * x[:, :, None, :])
    if not np.allclose(g["ddelta"], want, rtol=1e-12, atol=1e-12):
        return "ddelta differs from sum_n g_t (A h0 + B_t x_t)"
    assert L > 1
    return None


def pin_linearity(bwd):
    x, delta, A, B, C, h0, dy, dhT = _inputs(5)
    _, _, _, _, _, _, dy2, dhT2 = _inputs(6)
    g1 = bwd(x, delta, A, B, C, dy, h0, dhT)
    g2 = bwd(x, delta, A, B, C, dy2, h0, dhT2)
    g3 = bwd(x, delta, A, B, C, 2.0 * dy - 3.0 * dy2, h0, 2.0 * dhT - 3.0 * dhT2)
    for k in g1:
        if not np.allclose(g3[k], 2.0 * g1[k] - 3.0 * g2[k], rtol=1e-10, atol=1e-10):
            return f"{k} is not linear in (dy, dhT)"
    return None


def pin_reduces_to_ssd(bwd):
    x, delta, A, B, C, h0, dy, dhT = _inputs(7, N=3)
    A = np.repeat(A[:, :1], A.shape[1], axis=1)
    g = bwd(x, delta, A, B, C, dy, h0, dhT)
    ref = ssd_bwd_sequential(x.transpose(0, 2, 1)[..., None], delta.transpose(0, 2, 1), A[:, 0],
                             B.transpose(0, 2, 1)[:, :, None, :], C.transpose(0, 2, 1)[:, :, None, :],
                             np.zeros(x.shape[1]), dy.transpose(0, 2, 1)[..., None], h0[:, :, None, :],
                             dhT[:, :, None, :])
    checks = [("dx", g["dx"], ref["dx"][..., 0].transpose(0, 2, 1)),
              ("ddelta", g["ddelta"], ref["ddt"].transpose(0, 2, 1)),
              ("dB", g["dB"], ref["dB"][:, :, 0, :].transpose(0, 2, 1)),
              ("dC", g["dC"], ref["dC"][:, :, 0, :].transpose(0, 2, 1)),
              ("dh0", g["dh0"], ref["dinit"][:, :, 0, :]),
              ("dA", g["dA"].sum(axis=1), ref["dA"])]
    for name, got, want in checks:
        if not np.allclose(got, want, rtol=1e-10, atol=1e-10):
            return f"{name} differs from the SSD gradient with headdim 1"
    return None


PINS = {"g1": pin_finite_differences, "g2": pin_closed_forms, "g3": pin_linearity, "g4": pin_reduces_to_ssd}


@pytest.mark.parametrize("pin", sorted(PINS))
def test_s6_bwd_oracle_pins(pin):
    assert PINS[pin](s6_bwd_sequential) is None


def test_s6_bwd_without_h0_or_dhT():
    x, delta, A, B, C, _, dy, _ = _inputs(8, with_h0=False)
    g = s6_bwd_sequential(x, delta, A, B, C, dy)
    z = np.zeros((x.shape[0], x.shape[1], A.shape[1]))
    g0 = s6_bwd_sequential(x, delta, A, B, C, dy, z, z)
    for k in g:
        assert np.allclose(g[k], g0[k], rtol=0, atol=0), k


# ------------------------------------------------------------------ mutants
MUTANTS = {
    "ddelta without the decay term": ("np.sum(g * (A[None] * a * hp + Bt * xt), axis=2)", "np.sum(g * (Bt * xt), axis=2)"),
    "dA from the state after the step": ("dA += np.sum(g * dlt * a * hp, axis=0)",
                                        "dA += np.sum(g * dlt * a * hs[t + 1], axis=0)"),
    "dhT dropped": ("g = np.zeros((bt, D, N)) if dhT is None else np.array(dhT, dtype=np.float64, copy=True)",
                    "g = np.zeros((bt, D, N))"),
    "adjoint decayed before use": ("        g = g + C[:, None, :, t] * dy[:, :, t, None]          # dL/dh_t, complete",
                                   "        g = a_all[t] * g + C[:, None, :, t] * dy[:, :, t, None]"),
    "dC from the entering state": ("dC[:, :, t] = np.einsum(\"bd,bdn->bn\", dy[:, :, t], hs[t + 1])",
                                   "dC[:, :, t] = np.einsum(\"bd,bdn->bn\", dy[:, :, t], hs[t])"),
    "dx without delta": ("dx[:, :, t] = np.sum(g * Bt * dlt, axis=2)", "dx[:, :, t] = np.sum(g * Bt, axis=2)"),
    "dB summed over states": ("dB[:, :, t] = np.sum(g * dlt * xt, axis=1)",
                              "dB[:, :, t] = np.sum(g * dlt * xt, axis=1).sum(axis=1, keepdims=True) + 0 * dB[:, :, t]"),
}


def _mutant(old, new):
    src = inspect.getsource(s6mod)
    assert src.count(old) == 1, old
    mod = types.ModuleType("mutant_s6")
    exec(compile(src.replace(old, new), "<mutant s6>", "exec"), mod.__dict__)
    return mod.s6_bwd_sequential


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_s6_bwd_mutant_caught(name):
    bwd = _mutant(*MUTANTS[name])
    assert any(pin(bwd) is not None for pin in PINS.values()), f"no pin rejects the mutant {name}"
