"""The decode step on the GPU against the fp64 step oracle.

Every call goes through the C ABI (mamba2_ssd_step via the Python binding).
Tolerances: y as the forward pass's (fp32 io: 1e-5 normwise; bf16 io:
1e-2 + 2e-2|ref| per element); the fp32 state always to 1e-5 normwise, since
its inputs enter exactly and it is computed and kept in fp32.
"""
import numpy as np
import pytest
import torch

import state_space_sequence_ssd_amd as ssd
from oracle import ssd_sequential, ssd_step
from tests.gpu_helpers import check_close, host, log, run, to_device
from workloads import config_by_name, generate

pytestmark = pytest.mark.gpu


def step_inputs(cfg):
    """One token of `cfg` (seqlen 1) as decode-step arrays, plus the state."""
    inp = generate(cfg)
    out = {k: inp[k][:, 0] for k in ("x", "dt", "B", "C")}
    for k in ("x", "B", "C"):
        if k + "_bits" in inp:
            out[k + "_bits"] = inp[k + "_bits"][:, 0]
    out["A"], out["D"] = inp["A"], inp["D"]
    st = inp["init_state"]
    out["state"] = np.zeros((cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate), np.float32) if st is None else st
    return out


def dev_step(inp, io):
    d = to_device({**inp, "init_state": inp["state"]}, io)
    d["state"] = d.pop("init_state").clone()
    return d


def check_step(cfg, tag):
    log(f"[step] {tag}: {cfg.batch}x{cfg.nheads}x{cfg.headdim}x{cfg.dstate} G={cfg.ngroups} io={cfg.io}")
    inp = step_inputs(cfg)
    d = dev_step(inp, cfg.io)
    y = ssd.ssd_step(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["state"])
    torch.cuda.synchronize()
    yr, sr = ssd_step(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["state"])
    log("  " + check_close(host(y), yr, cfg.io, "y"))
    log("  " + check_close(host(d["state"]), sr, "f32", "state"))


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [64, 128, 256])
@pytest.mark.parametrize("P,G,H,batch", [(64, 1, 4, 2), (128, 2, 6, 3), (3, 3, 3, 5), (100, 1, 2, 7)])
def test_step_matches_oracle(io, N, P, G, H, batch):
    cfg = config_by_name("decode-small").with_shape(batch=batch, nheads=H, headdim=P, dstate=N, ngroups=G, io=io,
                                                    seed=100 + N + P + G)
    check_step(cfg, f"P={P} N={N}")


def test_step_serving_shape():
    """The 256-sequence 2.7B-like decode step, every output checked."""
    check_step(config_by_name("mamba2-2.7b-decode"), "serving")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_then_steps(io):
    """A GPU forward call over T tokens followed by K GPU steps from its final
    state reproduces the sequential oracle over T + K tokens: each step's y is
    that token's output, the last state the final state."""
    T, K = 300, 4
    cfg = config_by_name("mamba2-2.7b").with_shape(batch=2, seqlen=T + K, nheads=3, io=io, seed=31,
                                                   init_sigma=0.1)
    log(f"[step] prefill {T} then {K} steps, io={io}")
    inp = generate(cfg)
    pre = {k: (v[:, :T] if k in ("x", "dt", "B", "C", "x_bits", "B_bits", "C_bits") else v) for k, v in inp.items()}
    d = to_device(pre, io)
    _, fin = run(d, cfg.chunk)
    state = fin.clone()
    ys = []
    for t in range(T, T + K):
        one = {k: inp[k][:, t] for k in ("x", "dt", "B", "C")}
        for k in ("x", "B", "C"):
            if k + "_bits" in inp:
                one[k + "_bits"] = inp[k + "_bits"][:, t]
        one["A"], one["D"], one["init_state"] = inp["A"], inp["D"], None
        s = to_device(one, io)
        ys.append(host(ssd.ssd_step(s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"], state)))
    torch.cuda.synchronize()
    yr, fr = ssd_sequential(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["init_state"])
    for i, t in enumerate(range(T, T + K)):
        log("  " + check_close(ys[i], yr[:, t], io, f"y[t={t}]"))
    log("  " + check_close(host(state), fr, "f32", "state"))


def test_dt_zero_holds_the_state_exactly():
    """dt = 0: exp(0) = 1 and the update vanishes, so the state comes back bit
    for bit (the page's remark that dt = 0 keeps the state)."""
    cfg = config_by_name("decode-small")
    inp = step_inputs(cfg)
    inp["dt"] = np.zeros_like(inp["dt"])
    d = dev_step(inp, cfg.io)
    before = d["state"].clone()
    y = ssd.ssd_step(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["state"])
    torch.cuda.synchronize()
    assert torch.equal(d["state"], before)
    yr, _ = ssd_step(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["state"])
    check_close(host(y), yr, "f32", "y")


def test_empty_batch_is_a_no_op():
    x = torch.empty((0, 4, 64), device="cuda:0")
    st = torch.empty((0, 4, 64, 128), device="cuda:0")
    B = torch.empty((0, 1, 128), device="cuda:0")
    y = ssd.ssd_step(x, torch.empty((0, 4), device="cuda:0"), torch.full((4,), -1.0, device="cuda:0"), B, B,
                     torch.zeros(4, device="cuda:0"), st)
    assert y.shape == (0, 4, 64)
