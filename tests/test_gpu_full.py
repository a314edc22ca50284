"""GPU parity at the full configuration sizes, in the launch configuration the
benchmark times.

The oracle cannot evaluate a whole 2.7B-like layer in seconds, so each test
checks every token of a seeded sample of (batch, head) slices against the
chunked fp64 oracle (exact for those slices), and checks properties that hold
at any size on the whole output (finite values; chained calls equal one call).
"""
import numpy as np
import pytest
import torch

from oracle import ssd_chunked
from tests.gpu_helpers import check_close, host, log, run, to_device
from workloads import CONFIGS, generate

pytestmark = pytest.mark.gpu


def _sample(cfg, n):
    r = np.random.Generator(np.random.PCG64(cfg.seed + 99))
    picks = {(0, 0), (cfg.batch - 1, cfg.nheads - 1)}
    while len(picks) < n:
        picks.add((int(r.integers(cfg.batch)), int(r.integers(cfg.nheads))))
    return sorted(picks)


@pytest.mark.parametrize("cfg", CONFIGS, ids=[c.name for c in CONFIGS])
def test_full_config_sampled_heads(cfg):
    log(f"[full] {cfg.name}: generating inputs")
    inp = generate(cfg)
    dev = to_device(inp, cfg.io)
    log(f"[full] {cfg.name}: GPU call")
    y, fin = run(dev, cfg.chunk)
    assert bool(torch.isfinite(y.float()).all()) and bool(torch.isfinite(fin).all())
    picks = _sample(cfg, 4 if cfg.nheads * cfg.batch > 4 else cfg.nheads * cfg.batch)
    for b, h in picks:
        yr, fr = ssd_chunked(inp["x"][b:b + 1], inp["dt"][b:b + 1], inp["A"], inp["B"][b:b + 1],
                             inp["C"][b:b + 1], inp["D"], cfg.chunk,
                             None if inp["init_state"] is None else inp["init_state"][b:b + 1], heads=[h])
        log("  " + check_close(host(y[b:b + 1, :, h:h + 1]), yr, cfg.io, f"y[b={b},h={h}]"))
        log("  " + check_close(host(fin[b:b + 1, h:h + 1]), fr, cfg.io, f"final[b={b},h={h}]"))


def test_long_prefill_chained_in_eight_calls_equals_one_call():
    """The one-GPU stand-in for sequence sharding: eight calls of 8192 tokens,
    each starting from the previous final state, give bit-identical y and final
    state to one call over all 65536 tokens."""
    cfg = [c for c in CONFIGS if c.name == "long-prefill"][0]
    inp = generate(cfg)
    dev = to_device(inp, cfg.io)
    y, fin = run(dev, cfg.chunk)
    state = dev["init_state"]
    pieces = []
    seg = cfg.seqlen // 8
    for i in range(8):
        sl = slice(i * seg, (i + 1) * seg)
        d = {k: (v[:, sl].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in dev.items()}
        d["init_state"] = state
        yi, state = run(d, cfg.chunk)
        pieces.append(yi)
    assert torch.equal(torch.cat(pieces, dim=1), y)
    assert torch.equal(state, fin)
