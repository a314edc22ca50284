"""Pins for the backward-pass oracles (CPU only).

The gradients are tied to things fixed outside ``oracle/ssd_bwd.py``:

* b1 -- central finite differences of the forward oracle ``ssd_sequential``
  (itself pinned in test_oracle_pins.py): the gradient of the scalar loss
  sum(dy * y) + sum(dfinal * final) with respect to every input element is
  its definition.
* b2 -- closed forms: dD_h = sum over (b, t, p) of dy * x; with dt = 0 the
  state never moves, so dinit = dfinal + sum_t dy_t C_t^T, dx = D dy, dB = 0
  and dA = 0.
* b3 -- linearity: the gradients are linear in (dy, dfinal) jointly.
* b4 -- the two oracles (token recurrence, chunked) agree for every chunk
  length, ragged tails included.

Mutants planted in copies of both oracles must each fail b1-b3 (b4, the
cross-check, is left out of that test on purpose).
"""
import os
import types

import numpy as np
import pytest

from oracle import ssd_sequential
from oracle.ssd_bwd import ssd_bwd_chunked, ssd_bwd_sequential

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
NAMES = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "init": "dinit"}


def _problem(seed=0, bt=1, T=8, H=4, P=2, N=2, G=2, init=True, dfinal=True):
    rng = np.random.default_rng(seed)
    p = dict(x=rng.standard_normal((bt, T, H, P)), B=rng.standard_normal((bt, T, G, N)),
             C=rng.standard_normal((bt, T, G, N)),
             dt=np.log1p(np.exp(rng.standard_normal((bt, T, H)) - 1.0)),
             A=-np.exp(rng.uniform(0.0, 1.5, H)), D=rng.standard_normal(H),
             init=rng.standard_normal((bt, H, P, N)) if init else None)
    dy = rng.standard_normal((bt, T, H, P))
    dfin = rng.standard_normal((bt, H, P, N)) if dfinal else None
    return p, dy, dfin


def _seq(mod_seq):
    return lambda p, dy, dfin: mod_seq(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], dy, p["init"], dfin)


def _chunked(mod_chunked, Q):
    return lambda p, dy, dfin: mod_chunked(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], dy, Q, p["init"], dfin)


def _loss(p, dy, dfin):
    y, f = ssd_sequential(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["init"])
    return np.sum(y * dy) + (0.0 if dfin is None else np.sum(f * dfin))


def pin_finite_differences(bwd, seed=0, **shape):
    p, dy, dfin = _problem(seed, **shape)
    g = bwd(p, dy, dfin)
    eps = 1e-6
    for name, gname in NAMES.items():
        a = p[name]
        if a is None:
            continue
        fd = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            old = a[idx]
            a[idx] = old + eps
            lp = _loss(p, dy, dfin)
            a[idx] = old - eps
            lm = _loss(p, dy, dfin)
            a[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        err = np.abs(fd - g[gname]).max() / max(np.abs(fd).max(), 1e-300)
        if not err < 1e-6:
            return f"{gname}: finite-difference mismatch {err:.2e}"
    return None


def pin_closed_forms(bwd):
    p, dy, dfin = _problem(1)
    g = bwd(p, dy, dfin)
    dD = np.einsum("bthp,bthp->h", dy, p["x"])
    if not np.allclose(g["dD"], dD, rtol=1e-12, atol=1e-12):
        return "dD is not sum(dy * x)"
    # dt = 0: the state holds, y_t = init C_t + D x_t
    p["dt"][:] = 0.0
    g = bwd(p, dy, dfin)
    H, G = p["x"].shape[2], p["B"].shape[2]
    grp = np.arange(H) // (H // G)
    dinit = dfin + np.einsum("bthp,bthn->bhpn", dy, p["C"][:, :, grp])
    checks = [("dinit", dinit), ("dx", p["D"][None, None, :, None] * dy), ("dB", np.zeros_like(p["B"])),
              ("dA", np.zeros_like(p["A"]))]
    for name, want in checks:
        if not np.allclose(g[name], want, rtol=1e-12, atol=1e-12):
            return f"dt = 0: {name} differs from its closed form"
    return None


def pin_linearity(bwd):
    p, dy1, df1 = _problem(2)
    _, dy2, df2 = _problem(3)
    g1, g2 = bwd(p, dy1, df1), bwd(p, dy2, df2)
    g12 = bwd(p, dy1 + 2.0 * dy2, df1 + 2.0 * df2)
    for k in g1:
        want = g1[k] + 2.0 * g2[k]
        if not np.allclose(g12[k], want, rtol=1e-10, atol=1e-10 * max(1.0, np.abs(want).max())):
            return f"{k} is not linear in (dy, dfinal)"
    return None


BWD_PINS = [pin_finite_differences, pin_closed_forms, pin_linearity]


@pytest.mark.parametrize("which", ["sequential", "chunked-3", "chunked-4"])
@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda f: f.__name__)
def test_bwd_oracle_pins(pin, which):
    bwd = _seq(ssd_bwd_sequential) if which == "sequential" else _chunked(ssd_bwd_chunked, int(which[-1]))
    assert pin(bwd) is None


def test_bwd_finite_differences_without_init_or_dfinal():
    bwd = _seq(ssd_bwd_sequential)
    assert pin_finite_differences(bwd, seed=5, init=False, dfinal=False) is None
    assert pin_finite_differences(_chunked(ssd_bwd_chunked, 3), seed=5, init=False, dfinal=False) is None


@pytest.mark.parametrize("Q", [1, 2, 3, 5, 13, 16, 64])
def test_bwd_chunked_equals_sequential(Q):
    p, dy, dfin = _problem(4, bt=2, T=13, H=4, P=3, N=2, G=2)
    gs = _seq(ssd_bwd_sequential)(p, dy, dfin)
    gc = _chunked(ssd_bwd_chunked, Q)(p, dy, dfin)
    for k in gs:
        err = np.abs(gc[k] - gs[k]).max() / max(np.abs(gs[k]).max(), 1e-300)
        assert err < 1e-12, (k, Q, err)


# ------------------------------------------------------------------ mutants

SEQ_BWD_MUTANTS = {
    "skip_grad_dropped": ('out["dx"][b, t, h] += D[h] * dyt + dtt * (dh @ Bt)',
                          'out["dx"][b, t, h] += dtt * (dh @ Bt)'),
    "output_grad_scaled_by_decay": ("dh = dh + np.outer(dyt, Ct)", "dh = dh + alpha[t] * np.outer(dyt, Ct)"),
    "dalpha_uses_new_state": ("dalpha = np.sum(dh * states[t])", "dalpha = np.sum(dh * states[t + 1])"),
    "dA_without_dt": ('out["dA"][h] += dalpha * alpha[t] * dtt', 'out["dA"][h] += dalpha * alpha[t]'),
    "dB_without_dt": ('out["dB"][b, t, g] += dtt * (xt @ dh)', 'out["dB"][b, t, g] += xt @ dh'),
    "dC_reads_old_state": ('out["dC"][b, t, g] += dyt @ states[t + 1]', 'out["dC"][b, t, g] += dyt @ states[t]'),
    "dfinal_ignored": ("dh = np.zeros((P, N)) if dfinal is None else _f64(dfinal)[b, h].copy()",
                       "dh = np.zeros((P, N))"),
    "ddt_misses_decay_path": ("out[\"ddt\"][b, t, h] += xt @ dh @ Bt + dalpha * alpha[t] * a",
                              "out[\"ddt\"][b, t, h] += xt @ dh @ Bt"),
}

CHUNK_BWD_MUTANTS = {
    "dG_column_sign": ("- Z.sum(axis=0) - w * bvec", "+ Z.sum(axis=0) - w * bvec"),
    "carried_state_grad_undecayed": ("dHn = np.exp(Gl) * dHn + dYk.T @ (E[:, None] * Ck)",
                                     "dHn = dHn + dYk.T @ (E[:, None] * Ck)"),
    "dC_state_term_undecayed": ("dCh = W2 @ Bk + E[:, None] * (dYk @ Hprev[k])", "dCh = W2 @ Bk + (dYk @ Hprev[k])"),
    "ddt_forward_cumsum": ("ddt = ddt_direct + a * np.cumsum(dG[::-1])[::-1]", "ddt = ddt_direct + a * np.cumsum(dG)"),
    "mask_drops_diagonal": ("causal = np.tril(np.ones((Q, Q), dtype=bool))",
                            "causal = np.tril(np.ones((Q, Q), dtype=bool), -1)"),
    "dx_state_term_without_dt": ("dx = W1.T @ dYk + w[:, None] * dHnB + D[h] * dYk",
                                 "dx = W1.T @ dYk + np.exp(Gl - Gk)[:, None] * dHnB + D[h] * dYk"),
    "last_token_term_dropped": ("dG[-1] += np.exp(Gl) * np.sum(dHn * Hprev[k]) + np.sum(w * bvec)",
                                "dG[-1] += np.sum(w * bvec)"),
}


def _mutant(old, new):
    with open(os.path.join(ORACLE_DIR, "ssd_bwd.py")) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    src = src.replace(old, new).replace("from .ssd_seq import heads_to_groups",
                                        "from oracle.ssd_seq import heads_to_groups")
    mod = types.ModuleType("mutant_bwd")
    exec(compile(src, "<mutant bwd>", "exec"), mod.__dict__)
    return mod


def _caught(bwd):
    for pin in BWD_PINS:
        try:
            if pin(bwd) is not None:
                return True
        except (FloatingPointError, ValueError, IndexError):
            return True
    return False


@pytest.mark.parametrize("name", sorted(SEQ_BWD_MUTANTS))
def test_sequential_bwd_mutant_caught(name):
    mod = _mutant(*SEQ_BWD_MUTANTS[name])
    assert _caught(_seq(mod.ssd_bwd_sequential)), f"no pin rejects the mutant {name}"


@pytest.mark.parametrize("name", sorted(CHUNK_BWD_MUTANTS))
def test_chunked_bwd_mutant_caught(name):
    mod = _mutant(*CHUNK_BWD_MUTANTS[name])
    assert _caught(_chunked(mod.ssd_bwd_chunked, 3)), f"no pin rejects the mutant {name}"
