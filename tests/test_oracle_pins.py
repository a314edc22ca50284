"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import numpy as np
import pytest

from oracle import ssd_chunked, ssd_sequential, ssd_step
from tests.oracle_pins import ALL_PINS, assert_close, rand_layer


def seq_fwd(x, dt, A, B, C, D, h0):
    return ssd_sequential(x, dt, A, B, C, D, h0)


def chunked_fwd(q):
    def f(x, dt, A, B, C, D, h0):
        return ssd_chunked(x, dt, A, B, C, D, q, h0)
    return f


def stepped_fwd(x, dt, A, B, C, D, h0):
    """A whole sequence as repeated decode steps: every forward pin then pins
    the step oracle too."""
    x = np.asarray(x)
    bt, T, H, P = x.shape
    N = np.asarray(B).shape[-1]
    s = np.zeros((bt, H, P, N)) if h0 is None else np.asarray(h0, dtype=np.float64)
    y = np.empty((bt, T, H, P))
    for t in range(T):
        y[:, t], s = ssd_step(x[:, t], np.asarray(dt)[:, t], A, np.asarray(B)[:, t], np.asarray(C)[:, t], D, s)
    return y, s


FWDS = {"sequential": seq_fwd, "chunked_q1": chunked_fwd(1), "chunked_q4": chunked_fwd(4),
        "chunked_q5": chunked_fwd(5), "chunked_q64": chunked_fwd(64), "stepped": stepped_fwd}


@pytest.mark.parametrize("pin", sorted(ALL_PINS))
@pytest.mark.parametrize("impl", sorted(FWDS))
def test_pin(pin, impl):
    ALL_PINS[pin](FWDS[impl])


# ---------------------------------------------------------------- p3
@pytest.mark.parametrize("T,q", [(12, 1), (12, 2), (12, 3), (12, 4), (12, 6), (12, 12),
                                 (13, 4), (13, 5), (13, 16), (1, 1), (1, 8), (31, 8)])
def test_chunked_equals_sequential(T, q):
    """p3: the chunk-wise jump evaluation reproduces the token-by-token
    recurrence for every chunk size, including ragged tails (zero padding)."""
    x, dt, A, B, C, D, h0 = rand_layer(30 + T + q, T=T, dt_zero_frac=0.1)
    ys, fs = ssd_sequential(x, dt, A, B, C, D, h0)
    yc, fc = ssd_chunked(x, dt, A, B, C, D, q, h0)
    assert_close(yc, ys, 1e-12, "y")
    assert_close(fc, fs, 1e-12, "final")


def test_intermediates_consistent():
    """p3 at the checkpoints: the state entering chunk k equals the sequential
    state after token k*Q - 1; the last chunk's jump lands on the final state."""
    x, dt, A, B, C, D, h0 = rand_layer(40, T=16)
    q = 4
    _, fc, inter = ssd_chunked(x, dt, A, B, C, D, q, h0, return_intermediates=True)
    for k in range(4):
        if k == 0:
            ref = h0
        else:
            _, ref = ssd_sequential(x[:, :k * q], dt[:, :k * q], A, B[:, :k * q], C[:, :k * q], D, h0)
        assert_close(inter["hprev"][:, :, k], ref, 1e-12, f"hprev {k}")
    Glast = inter["G"][:, :, -1]
    jump = np.exp(Glast)[..., None, None] * inter["hprev"][:, :, -1] + inter["states"][:, :, -1]
    assert_close(jump, fc, 1e-13, "last jump")


def test_kept_exponents_nonpositive():
    """p4: every exponent the causal mask keeps, G_i - G_j for i >= j inside a
    chunk, is <= 0, and so is G itself; this holds exactly in floating point
    because a sequential sum of non-positive terms can only decrease."""
    for seed in range(5):
        x, dt, A, B, C, D, h0 = rand_layer(50 + seed, T=37, dt_zero_frac=0.2)
        for q in (4, 8, 37):
            _, _, inter = ssd_chunked(x, dt, A, B, C, D, q, h0, return_intermediates=True)
            G = inter["G"]
            nc = G.shape[-1] // q
            Gc = G.reshape(G.shape[:-1] + (nc, q))
            assert np.all(Gc <= 0.0)
            diff = Gc[..., :, None] - Gc[..., None, :]
            keep = np.tril(np.ones((q, q), dtype=bool))
            assert np.all(diff[..., keep] <= 0.0)


def test_heads_subset_matches_full():
    x, dt, A, B, C, D, h0 = rand_layer(60, T=9, H=6, G=3)
    yf, ff = ssd_chunked(x, dt, A, B, C, D, 4, h0)
    ys, fs = ssd_chunked(x, dt, A, B, C, D, 4, h0, heads=[1, 4])
    assert_close(ys, yf[:, :, [1, 4]], 0, "chunked subset y")
    assert_close(fs, ff[:, [1, 4]], 0, "chunked subset final")
    ys, fs = ssd_sequential(x, dt, A, B, C, D, h0, heads=[5, 0])
    yq, fq = ssd_sequential(x, dt, A, B, C, D, h0)
    assert_close(ys, yq[:, :, [5, 0]], 0, "seq subset y")
    assert_close(fs, fq[:, [5, 0]], 0, "seq subset final")


def test_empty_sequence():
    x, dt, A, B, C, D, h0 = rand_layer(61, T=1)
    e = lambda a: a[:, :0]
    for f in (lambda *a: ssd_sequential(*a), lambda *a: ssd_chunked(*a[:6], 4, a[6])):
        y, fin = f(e(x), e(dt), A, e(B), e(C), D, h0)
        assert y.shape == (2, 0, 4, 3)
        assert np.array_equal(fin, h0)


# ---------------------------------------------------------------- decode step
def test_steps_equal_both_forward_oracles():
    """Chaining the step oracle over a sequence reproduces the sequential and
    the chunked oracles (an independent route for each)."""
    x, dt, A, B, C, D, h0 = rand_layer(70, T=11, H=6, G=3, dt_zero_frac=0.1)
    ys, fs = stepped_fwd(x, dt, A, B, C, D, h0)
    yq, fq = ssd_sequential(x, dt, A, B, C, D, h0)
    yc, fc = ssd_chunked(x, dt, A, B, C, D, 4, h0)
    assert_close(ys, yq, 1e-13, "y vs sequential")
    assert_close(fs, fq, 1e-13, "state vs sequential")
    assert_close(ys, yc, 1e-12, "y vs chunked")
    assert_close(fs, fc, 1e-12, "state vs chunked")


def test_step_continues_a_prefill():
    """A step from a forward call's final state gives the next token's output
    and state of a forward call one token longer."""
    x, dt, A, B, C, D, h0 = rand_layer(71, T=9)
    yp, fp = ssd_chunked(x[:, :8], dt[:, :8], A, B[:, :8], C[:, :8], D, 4, h0)
    y1, f1 = ssd_step(x[:, 8], dt[:, 8], A, B[:, 8], C[:, 8], D, fp)
    yf, ff = ssd_sequential(x, dt, A, B, C, D, h0)
    assert_close(y1, yf[:, 8], 1e-12, "next y")
    assert_close(f1, ff, 1e-12, "next state")


def test_step_leaves_its_input_state_alone():
    x, dt, A, B, C, D, h0 = rand_layer(72, T=1)
    keep = h0.copy()
    ssd_step(x[:, 0], dt[:, 0], A, B[:, 0], C[:, 0], D, h0)
    assert np.array_equal(h0, keep)
