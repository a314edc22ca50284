"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one of them.

Each mutant is the oracle's own source with one textual edit, loaded into a
fresh module. A mutant that no pin rejects would mean the pins leave that part
of the oracle unchecked. The cross-check between the two oracles (p3) is left
out on purpose: every mutant must be caught by a pin that is independent of
the other oracle.
"""
import importlib.util
import os
import sys
import types

import pytest

from tests.oracle_pins import ALL_PINS

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

SEQ_MUTANTS = {
    "skip_sign": ("+ Ds[None, :, None] * xs[:, t]", "- Ds[None, :, None] * xs[:, t]"),
    "decay_sign": ("decay = np.exp(As[None, :] * step)", "decay = np.exp(-As[None, :] * step)"),
    "no_dt_on_key": ("b_t = step[:, :, None] * Bs[:, t]", "b_t = Bs[:, t]"),
    "group_modulo": ("np.arange(nheads) // (nheads // ngroups)", "np.arange(nheads) % ngroups"),
    "state_transposed": ("xs[:, t, :, :, None] * b_t[:, :, None, :]",
                         "(xs[:, t, :, :, None] * b_t[:, :, None, :]).transpose(0, 1, 3, 2)"),
    "y_reads_previous_state": ("        h = decay[:, :, None, None] * h +",
                               "        h_old = h\n        h = decay[:, :, None, None] * h +"),
    "decay_squared": ("decay[:, :, None, None] * h", "decay[:, :, None, None] ** 2 * h"),
}
# the y_reads_previous_state mutant needs its second half: y uses h_old
SEQ_FOLLOWUP = {"y_reads_previous_state": ('np.einsum("bhpn,bhn->bhp", h,', 'np.einsum("bhpn,bhn->bhp", h_old,')}

CHUNK_MUTANTS = {
    "mask_drops_diagonal": ("causal = np.tril(np.ones((chunk, chunk), dtype=bool))",
                            "causal = np.tril(np.ones((chunk, chunk), dtype=bool), -1)"),
    "glast_off_by_one": ("Glast = Gk[:, -1]", "Glast = Gk[:, -2]"),
    "carried_state_not_decayed": ("h = np.exp(Glast)[:, None, None] * h + Sk", "h = h + Sk"),
    "state_term_not_decayed": ("np.exp(Gk)[:, :, None] * np.matmul(Ck, h.transpose(0, 2, 1))",
                               "np.matmul(Ck, h.transpose(0, 2, 1))"),
    "state_contrib_without_dt": ("w = np.exp(Glast[:, None] - Gk) * dtk", "w = np.exp(Glast[:, None] - Gk)"),
    "exclusive_cumsum": ("Gk = np.cumsum(As[:, None] * dtk, axis=1)",
                         "Gk = np.cumsum(As[:, None] * dtk, axis=1) - As[:, None] * dtk"),
    "output_without_dt": ("dX = dtk[:, :, None] * Xk", "dX = Xk"),
    "skip_dropped": ("+ Ds[:, None, None] * Xk)", ")"),
    "decay_sign_flipped": ("expo = Gk[:, :, None] - Gk[:, None, :]", "expo = Gk[:, None, :] - Gk[:, :, None]"),
}


STEP_MUTANTS = {
    "decay_sign": ("alpha = np.exp(A[h] * dt[b, h])", "alpha = np.exp(-A[h] * dt[b, h])"),
    "no_dt_on_update": ("upd = np.outer(x[b, h], B[b, g]) * dt[b, h]", "upd = np.outer(x[b, h], B[b, g])"),
    "update_transposed": ("upd = np.outer(x[b, h], B[b, g]) * dt[b, h]",
                          "upd = np.outer(x[b, h], B[b, g]).T.reshape(x.shape[2], -1) * dt[b, h]"),
    "group_modulo": ("g = h // per_group", "g = h % G"),
    "y_reads_old_state": ("y[b, h] = s @ C[b, g]", "y[b, h] = state[b, h] @ C[b, g]"),
    "skip_dropped": ("+ D[h] * x[b, h]", "+ 0.0 * x[b, h]"),
    "y_contracts_B": ("y[b, h] = s @ C[b, g]", "y[b, h] = s @ B[b, g]"),
}


def _load_mutant(fname, modname, old, new, followup=None):
    with open(os.path.join(ORACLE_DIR, fname)) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique in {fname}: {old!r}"
    src = src.replace(old, new)
    if followup:
        assert src.count(followup[0]) == 1
        src = src.replace(*followup)
    # the chunked file imports heads_to_groups from the package; give it a fresh
    # package so a mutant never leaks into the real oracle modules
    pkg = types.ModuleType("mutant_oracle")
    pkg.__path__ = [ORACLE_DIR]
    sys.modules["mutant_oracle"] = pkg
    seq_spec = importlib.util.spec_from_file_location("mutant_oracle.ssd_seq", os.path.join(ORACLE_DIR, "ssd_seq.py"))
    seq_mod = importlib.util.module_from_spec(seq_spec)
    if fname == "ssd_seq.py":
        exec(compile(src, f"<mutant {modname}>", "exec"), seq_mod.__dict__)
    else:
        seq_spec.loader.exec_module(seq_mod)
    sys.modules["mutant_oracle.ssd_seq"] = seq_mod
    if fname == "ssd_seq.py":
        return seq_mod
    mod = types.ModuleType("mutant_oracle.ssd_chunked")
    mod.__package__ = "mutant_oracle"
    exec(compile(src, f"<mutant {modname}>", "exec"), mod.__dict__)
    return mod


def _caught(fwd):
    failed = []
    for name, pin in ALL_PINS.items():
        try:
            pin(fwd)
        except Exception as e:  # AssertionError, or a crash from broken shapes
            failed.append((name, type(e).__name__))
    return failed


@pytest.mark.parametrize("name", sorted(SEQ_MUTANTS))
def test_sequential_mutant_caught(name):
    mod = _load_mutant("ssd_seq.py", name, *SEQ_MUTANTS[name], followup=SEQ_FOLLOWUP.get(name))
    failed = _caught(lambda x, dt, A, B, C, D, h0: mod.ssd_sequential(x, dt, A, B, C, D, h0))
    assert failed, f"no pin rejects the sequential mutant {name}"


@pytest.mark.parametrize("q", [1, 4])
@pytest.mark.parametrize("name", sorted(CHUNK_MUTANTS))
def test_chunked_mutant_caught(name, q):
    mod = _load_mutant("ssd_chunked.py", name, *CHUNK_MUTANTS[name])
    failed = _caught(lambda x, dt, A, B, C, D, h0: mod.ssd_chunked(x, dt, A, B, C, D, q, h0))
    # a Q = 1 chunk has no off-diagonal and its last token is its only token,
    # so some mutants are genuinely invisible there; Q = 4 must catch them all
    if q == 1 and name in ("mask_drops_diagonal", "decay_sign_flipped", "glast_off_by_one"):
        return
    assert failed, f"no pin rejects the chunked mutant {name} at chunk {q}"


def test_unmutated_oracle_passes_every_pin():
    mod = _load_mutant("ssd_chunked.py", "identity", "Glast = Gk[:, -1]", "Glast = Gk[:, -1]")
    assert not _caught(lambda x, dt, A, B, C, D, h0: mod.ssd_chunked(x, dt, A, B, C, D, 4, h0))


@pytest.mark.parametrize("name", sorted(STEP_MUTANTS))
def test_step_mutant_caught(name):
    import numpy as np
    old, new = STEP_MUTANTS[name]
    with open(os.path.join(ORACLE_DIR, "ssd_step.py")) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("mutant_step")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)

    def stepped(x, dt, A, B, C, D, h0):
        x = np.asarray(x)
        bt, T, H, P = x.shape
        N = np.asarray(B).shape[-1]
        st = np.zeros((bt, H, P, N)) if h0 is None else np.asarray(h0, dtype=np.float64)
        y = np.empty((bt, T, H, P))
        for t in range(T):
            y[:, t], st = mod.ssd_step(x[:, t], np.asarray(dt)[:, t], A, np.asarray(B)[:, t],
                                       np.asarray(C)[:, t], D, st)
        return y, st

    assert _caught(stepped), f"no pin rejects the step mutant {name}"
