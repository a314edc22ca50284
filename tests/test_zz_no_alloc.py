"""mamba2_ssd_fwd_noalloc (the forward pass with the library's own device
array as its workspace) against mamba2_ssd_fwd with a caller workspace: two
calls in a row, the second smaller, each bit-identical to the allocating
entry point and within the stated tolerance of the fp64 oracle."""
import numpy as np
import pytest
import torch

import state_space_sequence_ssd_amd as ssd
from oracle import ssd_chunked
from tests.gpu_helpers import check_close, host, log, run, to_device
from workloads import config_by_name, generate

pytestmark = pytest.mark.gpu

CASES = [
    config_by_name("mamba2-130m").with_shape(batch=2, seqlen=3 * 256 + 77, nheads=12, init_sigma=0.2),
    config_by_name("mamba2-130m").with_shape(batch=1, seqlen=300, nheads=4),        # smaller second call
]


def _noalloc(dev, cfg):
    x = dev["x"]
    io = ssd.BF16 if x.dtype == torch.bfloat16 else ssd.F32
    dims = ssd.Dims(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, cfg.chunk)
    assert ssd.workspace_bytes(dims, io) <= ssd.NOALLOC_MAX_WORKSPACE
    y = torch.full_like(x, float("nan"))
    fin = torch.full((cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate), float("nan"), device=x.device)
    init = dev["init_state"]
    ptr = lambda t: 0 if t is None else t.data_ptr()
    ssd.ssd_fwd_noalloc_ptr(dims, io, ptr(x), ptr(dev["dt"]), ptr(dev["A"]), ptr(dev["B"]), ptr(dev["C"]),
                            ptr(dev["D"]), ptr(init), ptr(y), ptr(fin),
                            torch.cuda.current_stream(x.device).cuda_stream)
    torch.cuda.synchronize()
    return y, fin


def test_noalloc_matches_allocating_entry_point_twice():
    for i, cfg in enumerate(CASES):
        log(f"[noalloc] call {i}: {cfg}")
        inp = generate(cfg)
        dev = to_device(inp, cfg.io)
        y, fin = _noalloc(dev, cfg)
        y_ref, f_ref = run(dev, cfg.chunk)
        assert torch.equal(y, y_ref), f"call {i}: y differs from mamba2_ssd_fwd"
        assert torch.equal(fin, f_ref), f"call {i}: final_state differs from mamba2_ssd_fwd"
        yr, fr = ssd_chunked(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], cfg.chunk,
                             inp["init_state"])
        log("  " + check_close(host(y), yr, cfg.io, "y (noalloc)"))
        log("  " + check_close(host(fin), fr, cfg.io, "final_state (noalloc)"))


def test_noalloc_rejects_a_workspace_beyond_its_array():
    d = ssd.Dims(4, 8192, 80, 64, 128, 1, 256)
    io = ssd.BF16 | ssd.PATH_FOUR
    assert ssd.workspace_bytes(d, io) > ssd.NOALLOC_MAX_WORKSPACE
    with pytest.raises(ssd.SsdError) as e:
        ssd.ssd_fwd_noalloc_ptr(d, io, 256, 256, 256, 256, 256, 256, 0, 1 << 40, 0, 0)
    assert e.value.status == -6
