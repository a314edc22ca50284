"""GPU parity at the full configuration sizes, in the launch configuration the
benchmark times.

Every (batch, head) slice of every configuration is compared element by
element against the chunked fp64 oracle, one batch row at a time (the oracle
streams over chunks, so host memory stays bounded); chained calls are checked
to equal one call bit for bit.
"""
import functools

import numpy as np
import pytest
import torch

import state_space_sequence_ssd_amd as ssd
from oracle import ssd_chunked
from tests.gpu_helpers import check_close, host, log, run, to_device
from workloads import CONFIGS, generate

pytestmark = pytest.mark.gpu


def _dims(cfg):
    return ssd.Dims(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, cfg.chunk)


@functools.lru_cache(maxsize=1)
def _inputs(name):
    cfg = [c for c in CONFIGS if c.name == name][0]
    return cfg, generate(cfg)


CHAINED_OK = [c for c in CONFIGS if c.io == "bf16" and c.headdim == 64 and c.chunk == 256 and c.dstate <= 128]


@pytest.mark.parametrize("cfg,path", [(c, 0) for c in CONFIGS] + [(c, ssd.PATH_CHAINED) for c in CHAINED_OK],
                         ids=[c.name for c in CONFIGS] + [c.name + "-chained" for c in CHAINED_OK])
def test_full_config_every_head(cfg, path):
    log(f"[full] {cfg.name}: generating inputs")
    cfg, inp = _inputs(cfg.name)
    dev = to_device(inp, cfg.io)
    log(f"[full] {cfg.name}: GPU call (path {ssd.fwd_path(_dims(cfg), (1 if cfg.io == 'bf16' else 0) | path):#x})")
    y, fin = run(dev, cfg.chunk, path=path)
    yg, fg = host(y), host(fin)
    del y, dev
    torch.cuda.empty_cache()
    for b in range(cfg.batch):
        log(f"[full] {cfg.name}: oracle, batch row {b} of {cfg.batch} (all {cfg.nheads} heads)")
        init = None if inp["init_state"] is None else inp["init_state"][b:b + 1]
        yr, fr = ssd_chunked(inp["x"][b:b + 1], inp["dt"][b:b + 1], inp["A"], inp["B"][b:b + 1],
                             inp["C"][b:b + 1], inp["D"], cfg.chunk, init)
        log("  " + check_close(yg[b:b + 1], yr, cfg.io, f"y[b={b}]"))
        log("  " + check_close(fg[b:b + 1], fr, cfg.io, f"final[b={b}]"))
        del yr, fr


def test_long_prefill_chained_in_eight_calls_equals_one_call():
    """The one-GPU stand-in for sequence sharding: eight calls of 8192 tokens,
    each starting from the previous final state, give bit-identical y and final
    state to one call over all 65536 tokens."""
    cfg, inp = _inputs("long-prefill")
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
