"""GPU parity of the Mamba-1 selective scan (mamba1_s6_fwd through the C ABI)
against the fp64 S6 oracle.

Tolerance: fp32 in and out, so y and the final state are compared normwise,
max|got - ref| / max|ref| <= 1e-5 per tensor (the forward's fp32 bar). The
parallel scan multiplies a chunk's 64 per-step decays as one exp of their
summed exponent and splits the sequence into chunks; both change only
rounding.
"""
import numpy as np
import pytest
import torch

import state_space_sequence_ssd_amd as ssd
from oracle import s6_sequential
from tests.gpu_helpers import host, log
from workloads import generate_s6, s6_config_by_name

pytestmark = pytest.mark.gpu

TOL = 1e-5

SMALL = s6_config_by_name("s6-small")
CASES = {
    "small-h0": SMALL,
    "page-small": s6_config_by_name("s6-page").with_shape(batch=2, seqlen=256, channels=96),
    "n1": SMALL.with_shape(dstate=1, seqlen=129, channels=64),
    "n2": SMALL.with_shape(dstate=2, seqlen=64, channels=300),
    "n8": SMALL.with_shape(dstate=8, seqlen=517, channels=257, h0_sigma=None),
    "n16": s6_config_by_name("s6-mamba1-130m").with_shape(batch=1, seqlen=333, channels=130),
    "one-token": SMALL.with_shape(seqlen=1),
    "vec-path": SMALL.with_shape(seqlen=4 * 97, channels=256, dstate=16),
    "n16-scalar": SMALL.with_shape(dstate=16, batch=3, seqlen=171, channels=70),   # lane pairs, 4-byte rows
}


def _dev(inp):
    return {k: (None if v is None else torch.from_numpy(np.ascontiguousarray(v)).to("cuda:0")) for k, v in inp.items()}


def _run(t, h0="default"):
    h = t["h0"] if h0 == "default" else h0
    y, hT = ssd.s6_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], h)
    torch.cuda.synchronize()
    return y, hT


def _close(got, ref, what):
    got, ref = host(got), np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rel = float(np.max(np.abs(got - ref))) / max(float(np.max(np.abs(ref))), 1e-30) if ref.size else 0.0
    assert rel <= TOL, f"{what}: normwise relative error {rel:.3e} > {TOL}"
    return rel


@pytest.mark.parametrize("name", sorted(CASES))
def test_s6_parity(name):
    cfg = CASES[name]
    log(f"[s6] {name} {cfg}")
    inp = generate_s6(cfg)
    y, hT = _run(_dev(inp))
    yr, hr = s6_sequential(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["h0"])
    log(f"  y {_close(y, yr, 'y'):.1e}, hT {_close(hT, hr, 'hT'):.1e}")


def test_s6_chaining_and_in_place_state():
    """Two calls (the second from the first's final state, updated in place)
    give one call's outputs."""
    inp = generate_s6(SMALL.with_shape(seqlen=200))
    t = _dev(inp)
    y, hT = _run(t)
    cut = 77
    part = lambda k, a, b: t[k][..., a:b].contiguous()
    state = t["h0"].clone()
    dims1 = ssd.S6Dims(SMALL.batch, cut, SMALL.channels, SMALL.dstate)
    y1 = torch.empty_like(part("x", 0, cut))
    ws = torch.empty(max(ssd.s6_workspace_bytes(ssd.S6Dims(SMALL.batch, 200, SMALL.channels, SMALL.dstate)), 1),
                     dtype=torch.uint8, device="cuda:0")
    ins1 = [part(k, 0, cut) for k in ("x", "delta")] + [t["A"]] + [part(k, 0, cut) for k in ("B", "C")]
    ssd.s6_fwd_ptr(dims1, *[a.data_ptr() for a in ins1], state.data_ptr(), y1.data_ptr(), state.data_ptr(),
                   ws.data_ptr(), ws.numel())
    dims2 = ssd.S6Dims(SMALL.batch, 200 - cut, SMALL.channels, SMALL.dstate)
    y2 = torch.empty_like(part("x", cut, 200))
    ins2 = [part(k, cut, 200) for k in ("x", "delta")] + [t["A"]] + [part(k, cut, 200) for k in ("B", "C")]
    ssd.s6_fwd_ptr(dims2, *[a.data_ptr() for a in ins2], state.data_ptr(), y2.data_ptr(), state.data_ptr(),
                   ws.data_ptr(), ws.numel())
    torch.cuda.synchronize()
    yc = torch.cat([y1, y2], -1)
    rel_y = float((yc - y).abs().max() / y.abs().max())
    rel_h = float((state - hT).abs().max() / hT.abs().max())
    assert rel_y <= TOL and rel_h <= TOL, (rel_y, rel_h)


def test_s6_empty():
    inp = generate_s6(SMALL.with_shape(seqlen=0))
    t = _dev(inp)
    y, hT = _run(t)
    assert y.numel() == 0 and torch.equal(hT, t["h0"])
    y0, h0 = _run(t, h0=None)
    assert torch.count_nonzero(h0) == 0
    inp = generate_s6(SMALL.with_shape(batch=0))
    y, hT = _run(_dev(inp))
    assert y.numel() == 0 and hT.numel() == 0


def test_s6_page_shape_sampled_channels():
    """The page's benchmark call at full size, as bench.py times it, checked
    on a sample of channels (each channel's scan is independent)."""
    cfg = s6_config_by_name("s6-page")
    log(f"[s6] full {cfg}")
    inp = generate_s6(cfg)
    y, hT = _run(_dev(inp))
    ds = np.array([0, 1, 255, 256, 511, 700, 1023])
    yr, hr = s6_sequential(inp["x"][:, ds], inp["delta"][:, ds], inp["A"][ds], inp["B"], inp["C"], None)
    log(f"  y {_close(y[:, ds], yr, 'y'):.1e}, hT {_close(hT[:, ds], hr, 'hT'):.1e}")


def test_s6_mamba1_130m_every_element():
    # the Mamba-1 130M-like layer (dstate 16: each channel's states on a lane
    # pair) against the oracle on every element of y and hT
    cfg = s6_config_by_name("s6-mamba1-130m")
    inp = generate_s6(cfg)
    y, hT = _run(_dev(inp))
    yr, hr = s6_sequential(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["h0"])
    log(f"  y {_close(y, yr, 'y'):.1e}, hT {_close(hT, hr, 'hT'):.1e}")
