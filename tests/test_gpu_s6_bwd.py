"""GPU parity of the selective scan's backward pass (mamba1_s6_bwd through the
C ABI) against the fp64 gradient oracle (oracle.s6.s6_bwd_sequential).

Tolerance: fp32 arithmetic throughout, compared normwise per gradient,
max|g - g_ref| / max|g_ref| <= 1e-5 (the forward's fp32 bar; measured:
at most 6e-7). The kernels split the sequence into
64-token chunks, combine a chunk's decays as one exp of their summed
exponent and recompute the states from checkpoints: all of that changes
only rounding. The longest fp32 sums: dA over every token of every batch
row (32768 terms at the page's size) and dB, dC over up to 1536 channels;
sqrt(32768) * 2^-24 is about 1.1e-5, with cancellation where the terms
change sign.
"""
import numpy as np
import pytest
import torch

import state_space_sequence_ssd_amd as ssd
from oracle.s6 import s6_bwd_sequential
from tests.gpu_helpers import host, log
from workloads import generate_s6, s6_config_by_name

pytestmark = pytest.mark.gpu

TOL = 1e-5

SMALL = s6_config_by_name("s6-small")
CASES = {
    "small-h0": SMALL,                                                       # ragged tokens and channels
    "page-small": s6_config_by_name("s6-page").with_shape(batch=2, seqlen=256, channels=96),
    "n1": SMALL.with_shape(dstate=1, seqlen=129, channels=64),
    "n2": SMALL.with_shape(dstate=2, seqlen=64, channels=300),
    "n8": SMALL.with_shape(dstate=8, seqlen=517, channels=257, h0_sigma=None),   # two passes of 4 states
    "n16": SMALL.with_shape(dstate=16, seqlen=300, channels=130),                 # four passes
    "n16-scalar": SMALL.with_shape(dstate=16, seqlen=171, channels=70),
    "one-token": SMALL.with_shape(seqlen=1),
    "vec-path": SMALL.with_shape(seqlen=4 * 97, channels=256),                 # 16-byte rows, ragged chunk
    "two-blocks": SMALL.with_shape(batch=3, seqlen=200, channels=600),
    "scalar-half": SMALL.with_shape(seqlen=237, channels=130),               # 4-byte rows, 13 tokens in the last half
    "n2-short-tail": SMALL.with_shape(dstate=2, seqlen=148, channels=70),    # last chunk within its first half
}


def _dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")


def _upstream(cfg, seed, with_dhT=True):
    r = np.random.default_rng(seed)
    dy = r.standard_normal((cfg.batch, cfg.channels, cfg.seqlen)).astype(np.float32)
    dhT = r.standard_normal((cfg.batch, cfg.channels, cfg.dstate)).astype(np.float32) if with_dhT else None
    return dy, dhT


def _run(inp, dy, dhT):
    t = {k: _dev(v) for k, v in inp.items()}
    g = ssd.s6_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], _dev(dy), t["h0"], _dev(dhT))
    torch.cuda.synchronize()
    return g


def _check(g, ref, what=""):
    out = []
    for k in ssd.S6_GRAD_NAMES:
        got = host(g[k])
        want = np.asarray(ref[k], dtype=np.float64)
        assert got.shape == want.shape, (k, got.shape, want.shape)
        assert np.all(np.isfinite(got)), f"{what} {k}: non-finite values"
        den = max(float(np.max(np.abs(want))), 1e-30) if want.size else 1.0
        rel = float(np.max(np.abs(got - want))) / den if want.size else 0.0
        out.append(f"{k} {rel:.1e}")
        assert rel <= TOL, f"{what} {k}: normwise relative error {rel:.3e} > {TOL}"
    return ", ".join(out)


def _ref(inp, dy, dhT):
    return s6_bwd_sequential(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], dy, inp["h0"], dhT)


@pytest.mark.parametrize("name", sorted(CASES))
def test_s6_bwd_parity(name):
    cfg = CASES[name]
    log(f"[s6 bwd] {name} {cfg}")
    inp = generate_s6(cfg)
    dy, dhT = _upstream(cfg, 100 + len(name))
    log("  " + _check(_run(inp, dy, dhT), _ref(inp, dy, dhT), name))


def test_s6_bwd_without_h0_or_dhT():
    cfg = SMALL.with_shape(h0_sigma=None)
    inp = generate_s6(cfg)
    dy, _ = _upstream(cfg, 7, with_dhT=False)
    log("  " + _check(_run(inp, dy, None), _ref(inp, dy, None), "no h0, no dhT"))


def test_s6_bwd_empty_sequence_and_batch():
    # no token: dA = 0, dh0 = dhT, the token-shaped gradients empty
    cfg = SMALL.with_shape(seqlen=0)
    inp = generate_s6(cfg)
    dy, dhT = _upstream(cfg, 8)
    g = _run(inp, dy, dhT)
    assert np.all(host(g["dA"]) == 0.0)
    assert np.array_equal(host(g["dh0"]), dhT)
    assert g["dx"].numel() == 0 and g["dB"].numel() == 0
    cfg = SMALL.with_shape(batch=0)
    inp = generate_s6(cfg)
    dy, dhT = _upstream(cfg, 9)
    g = _run(inp, dy, dhT)
    assert np.all(host(g["dA"]) == 0.0)


def test_s6_bwd_is_deterministic():
    cfg = SMALL.with_shape(batch=2, seqlen=400, channels=300)
    inp = generate_s6(cfg)
    dy, dhT = _upstream(cfg, 10)
    g1, g2 = _run(inp, dy, dhT), _run(inp, dy, dhT)
    for k in ssd.S6_GRAD_NAMES:
        assert np.array_equal(host(g1[k]), host(g2[k])), k


def test_s6_bwd_mamba1_130m_every_gradient():
    # a Mamba-1 130M-like layer (dstate 16, 1536 channels, batch 8, 2048
    # tokens) against the oracle on every element of every gradient
    cfg = s6_config_by_name("s6-mamba1-130m")
    inp = generate_s6(cfg)
    dy, dhT = _upstream(cfg, 12)
    log("  " + _check(_run(inp, dy, dhT), _ref(inp, dy, dhT), "130m-like"))


def test_s6_bwd_page_size_every_gradient():
    # the page's benchmark shape (batch 8, seqlen 2048, channels 1024, dstate
    # 4) against the oracle on every element of every gradient
    cfg = s6_config_by_name("s6-page")
    inp = generate_s6(cfg)
    dy, dhT = _upstream(cfg, 11)
    log("  " + _check(_run(inp, dy, dhT), _ref(inp, dy, dhT), "page size"))
