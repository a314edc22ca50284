"""GPU parity of the backward pass (mamba2_ssd_bwd through the C ABI) against
the fp64 gradient oracle.

Tolerance: every gradient accumulates in fp32, and where a product takes an
fp32 intermediate on the bf16 MFMA (bf16 io, headdim 64, chunk 256) that
operand is a bf16 (hi, lo) pair, about 2^-17 (7.6e-6) relative per element;
each gradient is compared normwise, max|g - g_ref| / max|g_ref| <= 1e-4 per
tensor. The longest fp32 sums are over a chunk's tokens times headdim or
dstate (up to 256 * 256 terms): sqrt(65536) * 2^-24 is about 1.5e-5; the
time gradient also subtracts row and column sums of the same blocks. dA is
one number per head summed over every token of every batch row from those
time gradients (32768 tokens at the 2.7B-like size), and partly cancels: it
gets 5e-4.
"""
import numpy as np
import pytest
import torch

import state_space_sequence_ssd_amd as ssd
from oracle import ssd_bwd_chunked
from tests.gpu_helpers import host, log, to_device
from workloads import LayerConfig, config_by_name, generate

pytestmark = pytest.mark.gpu

BWD_TOL = 1e-4
TOL = {"dA": 5e-4}

CASES = {
    "tiny-f32": config_by_name("tiny"),
    "tiny-ragged-f32": config_by_name("tiny").with_shape(batch=2, seqlen=200),
    "130m-small": config_by_name("mamba2-130m").with_shape(batch=2, seqlen=2 * 256 + 77, nheads=6),
    "2.7b-small-init": config_by_name("long-prefill").with_shape(seqlen=3 * 256 + 13, nheads=5),
    "grouped-small": config_by_name("grouped-wide").with_shape(batch=1, seqlen=2 * 128 + 50, nheads=8, ngroups=2),
    "q64-p128": LayerConfig("bwd-q64", batch=1, seqlen=150, nheads=4, headdim=128, dstate=64, ngroups=1, chunk=64,
                            io="bf16", seed=31, init_sigma=0.5),
}


def _upstream(cfg, seed, with_dfinal=True):
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal((cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim)).astype(np.float32)
    if cfg.io == "bf16":
        from workloads import round_to_bf16
        dy = round_to_bf16(dy)[0]
    dfin = rng.standard_normal((cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate)).astype(np.float32) \
        if with_dfinal else None
    return dy, dfin


def _run(cfg, inp, dy, dfin):
    dev = to_device(inp, cfg.io)
    tdt = torch.bfloat16 if cfg.io == "bf16" else torch.float32
    dy_t = torch.from_numpy(dy).to(tdt).to("cuda:0")
    df_t = None if dfin is None else torch.from_numpy(dfin).to("cuda:0")
    g = ssd.ssd_bwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], dy_t, cfg.chunk,
                    dev["init_state"], df_t)
    torch.cuda.synchronize()
    return g


def _check(g, ref, what=""):
    out = []
    for k in ssd.GRAD_NAMES:
        got = host(g[k])
        want = np.asarray(ref[k], dtype=np.float64)
        assert got.shape == want.shape, (k, got.shape, want.shape)
        assert np.all(np.isfinite(got)), f"{what} {k}: non-finite values"
        den = max(float(np.max(np.abs(want))), 1e-30) if want.size else 1.0
        rel = float(np.max(np.abs(got - want))) / den if want.size else 0.0
        out.append(f"{k} {rel:.1e}")
        tol = TOL.get(k, BWD_TOL)
        assert rel <= tol, f"{what} {k}: normwise relative error {rel:.3e} > {tol}"
    return ", ".join(out)


@pytest.mark.parametrize("name", sorted(CASES))
def test_bwd_parity(name):
    cfg = CASES[name]
    log(f"[bwd] {name} {cfg}")
    inp = generate(cfg)
    dy, dfin = _upstream(cfg, seed=100 + len(name))
    g = _run(cfg, inp, dy, dfin)
    ref = ssd_bwd_chunked(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], dy, cfg.chunk,
                          inp["init_state"], dfin)
    log("  " + _check(g, ref, name))


def test_bwd_without_dfinal_and_init():
    cfg = CASES["130m-small"].with_shape(seqlen=300)
    inp = generate(cfg)
    inp["init_state"] = None
    dy, _ = _upstream(cfg, seed=7, with_dfinal=False)
    g = _run(cfg, inp, dy, None)
    ref = ssd_bwd_chunked(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], dy, cfg.chunk, None, None)
    log("  " + _check(g, ref, "no init, no dfinal"))


def test_bwd_empty_sequence_and_batch():
    cfg = CASES["tiny-f32"].with_shape(batch=2, seqlen=0, init_sigma=0.5)
    inp = generate(cfg)
    dy, dfin = _upstream(cfg, seed=3)
    g = _run(cfg, inp, dy, dfin)
    # no tokens: the initial state's gradient is dfinal, the head sums are zero
    assert torch.equal(g["dinit"].cpu(), torch.from_numpy(dfin))
    assert torch.count_nonzero(g["dA"]) == 0 and torch.count_nonzero(g["dD"]) == 0
    cfg0 = CASES["tiny-f32"].with_shape(batch=0, seqlen=100)
    inp0 = generate(cfg0)
    dy0, df0 = _upstream(cfg0, seed=4)
    g0 = _run(cfg0, inp0, dy0, df0)
    assert torch.count_nonzero(g0["dA"]) == 0 and torch.count_nonzero(g0["dD"]) == 0


def test_bwd_is_deterministic():
    cfg = CASES["130m-small"]
    inp = generate(cfg)
    dy, dfin = _upstream(cfg, seed=9)
    g1 = _run(cfg, inp, dy, dfin)
    g2 = _run(cfg, inp, dy, dfin)
    for k in ssd.GRAD_NAMES:
        assert torch.equal(g1[k], g2[k]), f"{k} differs between two identical calls"


def test_bwd_headline_every_gradient():
    """The 2.7B-like layer at full size, as bench.py --bwd runs it: every
    gradient tensor against the oracle, normwise over the whole tensor as in
    the smaller cases. The oracle runs one batch row at a time (all 80 heads,
    so dB and dC, which sum over the heads of the group, are complete per
    row); dA and dD sum over the rows."""
    cfg = config_by_name("mamba2-2.7b").with_shape(init_sigma=0.2)
    log(f"[bwd] headline {cfg}")
    inp = generate(cfg)
    dy, dfin = _upstream(cfg, seed=11)
    g = _run(cfg, inp, dy, dfin)
    got = {k: host(g[k]) for k in ssd.GRAD_NAMES}
    err = {k: 0.0 for k in ssd.GRAD_NAMES}
    big = {k: 0.0 for k in ssd.GRAD_NAMES}
    sums = {"dA": 0.0, "dD": 0.0}
    for b in range(cfg.batch):
        r = slice(b, b + 1)
        log(f"[bwd] headline: oracle, batch row {b} of {cfg.batch}")
        ref = ssd_bwd_chunked(inp["x"][r], inp["dt"][r], inp["A"], inp["B"][r], inp["C"][r], inp["D"], dy[r],
                              cfg.chunk, inp["init_state"][r], dfin[r])
        for k in ("dx", "ddt", "dB", "dC", "dinit"):
            want = np.asarray(ref[k], dtype=np.float64)
            err[k] = max(err[k], float(np.max(np.abs(got[k][r] - want))))
            big[k] = max(big[k], float(np.max(np.abs(want))))
        for k in sums:
            sums[k] = sums[k] + np.asarray(ref[k], dtype=np.float64)
    for k in sums:
        err[k] = float(np.max(np.abs(got[k] - sums[k])))
        big[k] = float(np.max(np.abs(sums[k])))
    msg = []
    for k in ssd.GRAD_NAMES:
        rel = err[k] / max(big[k], 1e-30)
        msg.append(f"{k} {rel:.1e}")
        assert rel <= TOL.get(k, BWD_TOL), f"{k}: normwise relative error {rel:.3e}"
    log("  " + ", ".join(msg))
