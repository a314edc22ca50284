"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small variants of every configuration (several tiles, ragged tails), each
kernel's output read back from the documented workspace, every supported
(headdim, dstate, chunk, io) instantiation, and the method's degenerate cases.
"""
import numpy as np
import pytest
import torch

import state_space_sequence_ssd_amd as ssd
from oracle import ssd_chunked, ssd_sequential
from tests.gpu_helpers import check_close, host, log, run, to_device, workspace_views
from workloads import CONFIGS, HELD_OUT, LayerConfig, config_by_name, generate

pytestmark = pytest.mark.gpu

LOG2E = 1.0 / np.log(2.0)

SMALL = {
    "tiny": config_by_name("tiny"),
    "tiny-ragged": config_by_name("tiny").with_shape(batch=2, seqlen=200),
    "130m-small": config_by_name("mamba2-130m").with_shape(batch=2, seqlen=2 * 256 + 77, nheads=6),
    "2.7b-small": config_by_name("mamba2-2.7b").with_shape(batch=1, seqlen=3 * 256 + 13, nheads=5),
    "long-small": config_by_name("long-prefill").with_shape(seqlen=4 * 256 + 200, nheads=3),
    "grouped-small": config_by_name("grouped-wide").with_shape(batch=1, seqlen=2 * 128 + 50, nheads=16, ngroups=2),
    "held-out-small": HELD_OUT.with_shape(batch=1, seqlen=300),
}


def oracle_all(inp, cfg, intermediates=False):
    return ssd_chunked(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], cfg.chunk,
                       inp["init_state"], return_intermediates=intermediates)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_variant_parity(name):
    """Every kernel's output on the FOUR sequence (the only one that writes
    each intermediate to the workspace) against the oracle's intermediates."""
    cfg = SMALL[name]
    log(f"[parity] {name}: {cfg}")
    inp = generate(cfg)
    yr, fr, inter = oracle_all(inp, cfg, intermediates=True)
    dev = to_device(inp, cfg.io)
    y, fin, ws, L, dims = run(dev, cfg.chunk, keep_workspace=True, path=ssd.PATH_FOUR)
    io = 1 if cfg.io == "bf16" else 0
    v = workspace_views(ws, L, dims, io)
    Tp = L.nchunks * cfg.chunk
    T = cfg.seqlen

    # ssd_chunk_cumsum: G' = log2(e) * chunk-local cumsum, padded tokens repeat the last value
    g = host(v["gcum"])
    gref = inter["G"] * LOG2E
    scale = np.max(np.abs(gref), axis=-1, keepdims=True) + 1.0
    assert np.all(np.abs(g - gref) <= 4e-5 * scale), "gcum"
    dtt = v["dtt"].cpu().numpy()
    assert np.array_equal(dtt[:, :, :T], np.transpose(inp["dt"], (0, 2, 1))), "dtt"
    assert np.all(dtt[:, :, T:] == 0)
    # state weights: dt_t * exp(G_last - G_t) of the chunk. G' is fp32, so the
    # exponent G'_last - G'_t carries an absolute error of a few ulp(|G'|):
    # the bound on w is relative, growing with the magnitudes involved.
    Gr = inter["G"].reshape(cfg.batch, cfg.nheads, L.nchunks, cfg.chunk)
    dtp = np.zeros((cfg.batch, cfg.nheads, Tp))
    dtp[:, :, :T] = np.transpose(inp["dt"], (0, 2, 1))
    wref = (dtp.reshape(Gr.shape) * np.exp(Gr[..., -1:] - Gr)).reshape(dtp.shape)
    gmag = (np.abs(Gr[..., -1:]) + np.abs(Gr)).reshape(dtp.shape) * LOG2E
    wg = host(v["wst"])
    assert np.all(np.abs(wg - wref) <= (1e-5 + 8 * 2.0 ** -24 * gmag) * np.abs(wref) + 1e-30), "wst"
    # monotone within each chunk: every kept exponent is <= 0 exactly
    gc = v["gcum"].cpu().numpy().reshape(cfg.batch, cfg.nheads, L.nchunks, cfg.chunk)
    assert np.all(np.diff(gc, axis=-1) <= 0) and np.all(gc <= 0)

    # ssd_chunk_state and ssd_state_pass
    log("  " + check_close(host(v["states"]), inter["states"], cfg.io, "states"))
    log("  " + check_close(host(v["hprev"]), inter["hprev"], cfg.io, "hprev"))
    # ssd_chunk_scan
    log("  " + check_close(host(y), yr, cfg.io, "y"))
    log("  " + check_close(host(fin), fr, cfg.io, "final_state"))


def test_small_variant_matches_sequential_oracle():
    """The same GPU result against the token-by-token oracle."""
    cfg = SMALL["130m-small"]
    inp = generate(cfg)
    ys, fs = ssd_sequential(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["init_state"])
    y, fin = run(to_device(inp, cfg.io), cfg.chunk)
    check_close(host(y), ys, cfg.io, "y vs sequential")
    check_close(host(fin), fs, cfg.io, "final vs sequential")


SWEEP = [(P, N, Q, io) for P in (64, 128) for N in (64, 128, 256) for Q in (64, 128, 256) for io in ("f32", "bf16")]


@pytest.mark.parametrize("P,N,Q,io", SWEEP)
def test_every_instantiation(P, N, Q, io):
    cfg = LayerConfig(f"sweep-{P}-{N}-{Q}-{io}", batch=1, seqlen=2 * Q + 17, nheads=4, headdim=P, dstate=N,
                      ngroups=2, chunk=Q, io=io, seed=1000 + P + N + Q, init_sigma=0.5)
    log(f"[sweep] P={P} N={N} Q={Q} io={io}")
    inp = generate(cfg)
    yr, fr = oracle_all(inp, cfg)
    y, fin = run(to_device(inp, io), Q)
    check_close(host(y), yr, io, "y")
    check_close(host(fin), fr, io, "final_state")


# ------------------------------------------------------------------ edge cases

def _cfg(**kw):
    base = dict(batch=2, seqlen=300, nheads=4, headdim=64, dstate=128, ngroups=1, chunk=128, io="bf16",
                seed=77, init_sigma=0.3)
    base.update(kw)
    return LayerConfig("edge", **base)


@pytest.mark.parametrize("T", [0, 1, 5, 127, 128, 129])
def test_short_and_empty_sequences(T):
    cfg = _cfg(seqlen=T)
    log(f"[edge] seqlen={T}")
    inp = generate(cfg)
    dev = to_device(inp, cfg.io)
    y, fin = run(dev, cfg.chunk)
    yr, fr = oracle_all(inp, cfg)
    if T == 0:
        assert y.numel() == 0
        assert torch.equal(fin, dev["init_state"]), "seqlen 0 must return the initial state"
        y0, f0 = run(dev, cfg.chunk, init_state=None)
        assert torch.count_nonzero(f0) == 0
        return
    check_close(host(y), yr, cfg.io, "y")
    check_close(host(fin), fr, cfg.io, "final")


def test_dt_zero_holds_state_exactly():
    cfg = _cfg(seqlen=3 * 128 + 9)
    inp = generate(cfg)
    inp["dt"][:] = 0.0
    dev = to_device(inp, cfg.io)
    y, fin = run(dev, cfg.chunk)
    assert torch.equal(fin, dev["init_state"]), "dt == 0 must leave the state bit-identical"
    yr, _ = oracle_all(inp, cfg)
    check_close(host(y), yr, cfg.io, "y with dt == 0")


@pytest.mark.parametrize("io,chunk", [("f32", 128), ("bf16", 128), ("bf16", 256)])
def test_zero_decay_is_linear_attention(io, chunk):
    """A = 0 (the limit of the decay going away): causal linear attention,
    as one dense T x T masked product."""
    cfg = _cfg(seqlen=2 * chunk + 3, io=io, init_sigma=None, chunk=chunk, headdim=64)
    inp = generate(cfg)
    inp["A"][:] = 0.0
    y, fin = run(to_device(inp, cfg.io), cfg.chunk)
    x, dt, B, C, D = inp["x"], inp["dt"], inp["B"], inp["C"], inp["D"]
    T = cfg.seqlen
    mask = np.tril(np.ones((T, T)))
    ref = np.empty(x.shape)
    for b in range(cfg.batch):
        for h in range(cfg.nheads):
            Cg, Bg = C[b, :, 0].astype(np.float64), B[b, :, 0].astype(np.float64)
            X = x[b, :, h].astype(np.float64)
            ref[b, :, h] = ((Cg @ Bg.T) * mask) @ (dt[b, :, h, None] * X) + D[h] * X
    log("  " + check_close(host(y), ref, io, "linear attention"))


def test_in_place_state_update():
    cfg = _cfg()
    inp = generate(cfg)
    dev = to_device(inp, cfg.io)
    ref_y, ref_f = run(dev, cfg.chunk)
    state = dev["init_state"].clone()
    import state_space_sequence_ssd_amd as ssd
    y, f = ssd.ssd_fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], cfg.chunk, state,
                       final_state=state)
    torch.cuda.synchronize()
    assert f.data_ptr() == state.data_ptr()
    assert torch.equal(state, ref_f) and torch.equal(y, ref_y)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_chaining_at_chunk_boundaries_is_bit_exact(io):
    """One call over T tokens equals a call over the first T1 (a multiple of
    the chunk) followed by a call over the rest from its final state: the
    fp32 state carried between chunks is the same value either way."""
    cfg = _cfg(seqlen=5 * 128 + 40, io=io)
    inp = generate(cfg)
    dev = to_device(inp, io)
    y, fin = run(dev, cfg.chunk)
    T1 = 2 * 128
    part = lambda d, sl: {k: (v[:, sl].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in d.items()}
    y1, f1 = run(part(dev, slice(0, T1)), cfg.chunk)
    d2 = part(dev, slice(T1, None))
    d2["init_state"] = f1
    y2, f2 = run(d2, cfg.chunk)
    assert torch.equal(torch.cat([y1, y2], dim=1), y)
    assert torch.equal(f2, fin)


def test_deterministic_and_guard_bands():
    cfg = _cfg(seqlen=2 * 128 + 31, batch=1)
    inp = generate(cfg)
    dev = to_device(inp, cfg.io)
    import state_space_sequence_ssd_amd as ssd
    n_y = dev["x"].numel()
    n_f = dev["init_state"].numel()
    pad = 4096
    ybig = torch.full((n_y + 2 * pad,), float("nan"), dtype=torch.bfloat16, device="cuda")
    fbig = torch.full((n_f + 2 * pad,), float("nan"), dtype=torch.float32, device="cuda")
    L = ssd.workspace_layout(ssd.Dims(1, cfg.seqlen, 4, 64, 128, 1, 128), ssd.BF16)
    wbig = torch.full((L.total_bytes + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
    yv = ybig[pad:pad + n_y].view(dev["x"].shape)
    fv = fbig[pad:pad + n_f].view(dev["init_state"].shape)
    wv = wbig[pad:pad + L.total_bytes]
    outs = []
    for _ in range(2):
        ssd.ssd_fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], cfg.chunk, dev["init_state"],
                    y=yv, final_state=fv, workspace=wv)
        torch.cuda.synchronize()
        outs.append((yv.clone(), fv.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1]), "not deterministic"
    for big, name in ((ybig, "y"), (fbig, "final")):
        assert torch.all(torch.isnan(big[:pad])) and torch.all(torch.isnan(big[-pad:])), f"{name} canary written"
    assert torch.all(wbig[:pad] == 0xA5) and torch.all(wbig[-pad:] == 0xA5), "workspace canary written"
    yr, fr = oracle_all(inp, cfg)
    check_close(host(outs[0][0]), yr, cfg.io, "y")


def test_outputs_follow_the_stream():
    """The call is enqueued on torch's current stream: work on a side stream
    ordered after it sees the finished output."""
    cfg = _cfg()
    inp = generate(cfg)
    dev = to_device(inp, cfg.io)
    ref_y, _ = run(dev, cfg.chunk)
    s = torch.cuda.Stream()
    import state_space_sequence_ssd_amd as ssd
    with torch.cuda.stream(s):
        y, _ = ssd.ssd_fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], cfg.chunk,
                           dev["init_state"])
        z = y.float() * 1.0
    s.synchronize()
    assert torch.equal(z, ref_y.float())


# ---------------------------------------------- C.B^T-resident scan (bf16, P=64, Q=256, N in {64, 128})
# That kernel walks consecutive heads of a chunk per workgroup and keeps the
# chunk's C.B^T in registers; these cases drive its walk (ragged last
# chunks, chunk and group changes inside a workgroup's range, grids with and
# without the XCD grouping, fewer tiles than workgroups).
RESIDENT = {
    "T1": dict(batch=2, seqlen=1, nheads=3),
    "T200": dict(batch=2, seqlen=200, nheads=3),
    "T256": dict(batch=1, seqlen=256, nheads=5),
    "T257": dict(batch=2, seqlen=257, nheads=3),
    "T1000-N64": dict(batch=1, seqlen=1000, nheads=4, dstate=64),
    "groups-xcd": dict(batch=4, seqlen=2048, nheads=8, ngroups=2),
    "walk-crosses-chunks": dict(batch=1, seqlen=4096, nheads=24),
    "walk-ragged-xcd": dict(batch=8, seqlen=700, nheads=6, ngroups=3),
}


@pytest.mark.parametrize("name", sorted(RESIDENT))
def test_resident_scan_walks(name):
    cfg = LayerConfig(f"resident-{name}", **{**dict(headdim=64, dstate=128, ngroups=1, chunk=256, io="bf16",
                                                  seed=500 + len(name), init_sigma=0.2), **RESIDENT[name]})
    log(f"[resident] {name}: {cfg}")
    inp = generate(cfg)
    yr, fr = oracle_all(inp, cfg)
    dev = to_device(inp, cfg.io)
    y, fin = run(dev, cfg.chunk)
    log("  " + check_close(host(y), yr, cfg.io, "y"))
    log("  " + check_close(host(fin), fr, cfg.io, "final_state"))
    y2, _ = run(dev, cfg.chunk)
    assert torch.equal(y, y2), "two identical calls must give identical y"


# ------------------------------------ chunk states computed inside the state pass
# (bf16, dstate 128 or 256: the THREE sequence). The path field of io
# forces either sequence regardless of size; both must match the oracle, and
# each other up to fp32 rounding (the two forms sum a chunk's tokens in
# different orders).
# Two sequences store hprev as bf16 (hi, lo) pairs of fp32 states summed in
# different orders: each stored pair is within 2^-16 of its fp32 value (hi and
# lo both round to nearest), so the two may differ by about twice that.
HPREV_PAIR_TOL = 2.0 ** -15

FUSED = {
    "2.7b-ragged": dict(batch=2, seqlen=3 * 256 + 13, nheads=5),
    "one-chunk": dict(batch=3, seqlen=100, nheads=2),
    "N64": dict(batch=1, seqlen=5 * 256 + 1, nheads=4, dstate=64),
    "two-wave-form": dict(batch=2, seqlen=2 * 256 + 20, nheads=128),   # 512 walks: the two-wave form
    "P128-N256-Q128": dict(batch=1, seqlen=700, nheads=8, headdim=128, dstate=256, ngroups=2, chunk=128),
    "Q64": dict(batch=2, seqlen=5 * 64 + 9, nheads=3, chunk=64),
    "N256-groups": dict(batch=1, seqlen=600, nheads=8, dstate=256, ngroups=2),
    "exact-chunks": dict(batch=2, seqlen=4 * 256, nheads=3),
    "long-walk": dict(batch=1, seqlen=20 * 256 + 77, nheads=2),
}


@pytest.mark.parametrize("name", sorted(FUSED))
def test_fused_state_pass(name):
    cfg = LayerConfig(f"fused-{name}", **{**dict(headdim=64, dstate=128, ngroups=1, chunk=256, io="bf16",
                                               seed=700 + len(name), init_sigma=0.3), **FUSED[name]})
    log(f"[fused] {name}: {cfg}")
    inp = generate(cfg)
    yr, fr, inter = oracle_all(inp, cfg, intermediates=True)
    dev = to_device(inp, cfg.io)
    y1, f1, ws1, L, dims = run(dev, cfg.chunk, keep_workspace=True, path=ssd.PATH_THREE)
    assert ssd.fused_state_pass(dims, 1 | ssd.PATH_THREE) and L.path == ssd.PATH_THREE
    v = workspace_views(ws1, L, dims, 1)
    log("  " + check_close(host(v["hprev"]), inter["hprev"], cfg.io, "hprev (fused)"))
    log("  " + check_close(host(y1), yr, cfg.io, "y (fused)"))
    log("  " + check_close(host(f1), fr, cfg.io, "final_state (fused)"))
    y2, f2, ws2, L2, _ = run(dev, cfg.chunk, keep_workspace=True, path=ssd.PATH_FOUR)
    assert not ssd.fused_state_pass(dims, 1 | ssd.PATH_FOUR) and L2.path == ssd.PATH_FOUR
    v2 = workspace_views(ws2, L2, dims, 1)
    for what, a1, a2, tol in (("hprev", v["hprev"], v2["hprev"], HPREV_PAIR_TOL), ("final_state", f1, f2, 1e-5)):
        a1, a2 = host(a1), host(a2)
        rel = float(np.max(np.abs(a1 - a2))) / max(float(np.max(np.abs(a2))), 1e-30)
        assert rel <= tol, f"{what}: paths differ by {rel:.2e} (normwise)"
    # y: one bf16 ulp of each output, plus what the hprev difference above can
    # move it by where the carried-state and in-chunk terms cancel (2^-15 of a
    # term as large as the largest output, with margin)
    yy1, yy2 = host(y1), host(y2)
    ymax = float(np.max(np.abs(yy2)))
    assert np.all(np.abs(yy1 - yy2) <= 2.0 ** -7 * np.abs(yy2) + 2.0 ** -12 * ymax), \
        "y: paths differ by more than one bf16 ulp plus the hprev difference"


ROW_SWEEP = [(P, N, Q) for P in (64, 128) for N in (128, 256) for Q in (64, 128, 256)]


@pytest.mark.parametrize("P,N,Q", ROW_SWEEP)
def test_row_form_every_instantiation(P, N, Q):
    """The three-kernel sequence at small sizes runs the row form of the state
    pass (one workgroup per batch, head and 128-column dstate slice): every
    headdim, dstate and chunk it is built for, with a ragged last chunk, two
    groups and a nonzero initial state, against the oracle's hprev, y and
    final state."""
    cfg = LayerConfig(f"rows-{P}-{N}-{Q}", batch=1, seqlen=3 * Q + 17, nheads=4, headdim=P, dstate=N,
                      ngroups=2, chunk=Q, io="bf16", seed=1300 + P + N + Q, init_sigma=0.5)
    log(f"[rows] P={P} N={N} Q={Q}")
    inp = generate(cfg)
    yr, fr, inter = oracle_all(inp, cfg, intermediates=True)
    y, fin, ws, L, dims = run(to_device(inp, cfg.io), Q, keep_workspace=True, path=ssd.PATH_THREE)
    assert ssd.fused_state_pass(dims, 1 | ssd.PATH_THREE) and L.path == ssd.PATH_THREE
    v = workspace_views(ws, L, dims, 1)
    log("  " + check_close(host(v["hprev"]), inter["hprev"], cfg.io, "hprev (row form)"))
    log("  " + check_close(host(y), yr, cfg.io, "y"))
    log("  " + check_close(host(fin), fr, cfg.io, "final_state"))


def test_fused_state_pass_in_place_and_no_final():
    """init_state may be final_state (in-place update); final_state may be absent."""
    cfg = LayerConfig("fused-inplace", batch=2, seqlen=2 * 256 + 40, nheads=3, headdim=64, dstate=128,
                      ngroups=1, chunk=256, io="bf16", seed=731, init_sigma=0.3)
    inp = generate(cfg)
    yr, fr = oracle_all(inp, cfg)
    dev = to_device(inp, cfg.io)
    st = dev["init_state"].clone()
    y, fin = ssd.ssd_fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], cfg.chunk, st,
                         final_state=st, path=ssd.PATH_THREE)
    torch.cuda.synchronize()
    assert fin.data_ptr() == st.data_ptr()
    check_close(host(st), fr, cfg.io, "final_state in place (fused)")
    check_close(host(y), yr, cfg.io, "y (fused, in place)")
    y2, none = ssd.ssd_fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], cfg.chunk,
                           dev["init_state"], return_final_state=False, path=ssd.PATH_THREE)
    torch.cuda.synchronize()
    assert none is None
    check_close(host(y2), yr, cfg.io, "y (fused, no final)")


# --------------------------------- states, pass and outputs in one kernel
# (bf16, headdim 64, chunk 256, dstate 64/128: the CHAINED sequence). Each
# case is checked against the oracle and against the FOUR sequence, and the
# workspace's error word (set when a wait for the previous chunk's state hits
# its bound) must stay 0.
CHAINED = {
    "ragged-init": dict(batch=2, seqlen=3 * 256 + 13, nheads=5, init_sigma=0.3),
    "one-chunk": dict(batch=3, seqlen=100, nheads=2),
    "N64-groups": dict(batch=1, seqlen=5 * 256 + 1, nheads=8, dstate=64, ngroups=2, init_sigma=0.2),
    "exact-chunks": dict(batch=2, seqlen=4 * 256, nheads=6),
    "long-walk": dict(batch=1, seqlen=40 * 256 + 77, nheads=3, init_sigma=0.1),
    "many-heads": dict(batch=2, seqlen=6 * 256, nheads=48, init_sigma=0.1),
}


def _sync_error_word(ws, L):
    return int(ws[L.sync_offset + 8:L.sync_offset + 12].view(torch.int32).item())


@pytest.mark.parametrize("name", sorted(CHAINED))
def test_chained_sequence(name):
    cfg = LayerConfig(f"chained-{name}", **{**dict(headdim=64, dstate=128, ngroups=1, chunk=256, io="bf16",
                                                 seed=900 + len(name)), **CHAINED[name]})
    log(f"[chained] {name}: {cfg}")
    inp = generate(cfg)
    yr, fr = oracle_all(inp, cfg)
    dev = to_device(inp, cfg.io)
    y, fin, ws, L, dims = run(dev, cfg.chunk, keep_workspace=True, path=ssd.PATH_CHAINED)
    assert L.path == ssd.PATH_CHAINED
    assert L.states_offset == L.hprev_offset == L.chain_offset == L.wst_offset
    assert _sync_error_word(ws, L) == 0, "a wait for the previous chunk's state hit its bound"
    log("  " + check_close(host(y), yr, cfg.io, "y (chained)"))
    log("  " + check_close(host(fin), fr, cfg.io, "final_state (chained)"))
    y4, f4 = run(dev, cfg.chunk, path=ssd.PATH_FOUR)
    rel = float(torch.max(torch.abs(fin - f4))) / max(float(torch.max(torch.abs(f4))), 1e-30)
    assert rel <= 1e-5, f"final_state: CHAINED and FOUR differ by {rel:.2e} (normwise)"
    # the sequences sum in different orders (fp32), then round to bf16: at most
    # one bf16 ulp apart, plus an absolute floor for values near zero
    yy, y4h = host(y), host(y4)
    diff = np.abs(yy - y4h)
    bound = 2.0 ** -7 * np.abs(y4h) + 1e-5 * float(np.max(np.abs(y4h)))
    i = np.unravel_index(int(np.argmax(diff / bound)), diff.shape)
    assert np.all(diff <= bound), (f"y: CHAINED and FOUR differ beyond one bf16 ulp: worst at {i}: "
                                   f"{yy[i]:.6g} vs {y4h[i]:.6g} (max|y| {float(np.max(np.abs(y4h))):.3g})")
    y2, f2 = run(dev, cfg.chunk, path=ssd.PATH_CHAINED)
    assert torch.equal(y, y2) and torch.equal(fin, f2), "two identical calls must give identical results"


def test_chained_in_place_and_no_final():
    cfg = LayerConfig("chained-inplace", batch=2, seqlen=2 * 256 + 40, nheads=3, headdim=64, dstate=128,
                      ngroups=1, chunk=256, io="bf16", seed=931, init_sigma=0.3)
    inp = generate(cfg)
    yr, fr = oracle_all(inp, cfg)
    dev = to_device(inp, cfg.io)
    st = dev["init_state"].clone()
    y, fin = ssd.ssd_fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], cfg.chunk, st,
                         final_state=st, path=ssd.PATH_CHAINED)
    torch.cuda.synchronize()
    assert fin.data_ptr() == st.data_ptr()
    check_close(host(st), fr, cfg.io, "final_state in place (chained)")
    check_close(host(y), yr, cfg.io, "y (chained, in place)")
    y2, none = ssd.ssd_fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], cfg.chunk,
                           dev["init_state"], return_final_state=False, path=ssd.PATH_CHAINED)
    torch.cuda.synchronize()
    assert none is None
    check_close(host(y2), yr, cfg.io, "y (chained, no final)")


# ------------------------------------------------------------ dt layouts

DT_LAYOUT = {
    "tiny": SMALL["tiny"],                     # f32, full chunks, T % 4 == 0 (16-byte dt reads)
    "tiny-ragged": SMALL["tiny-ragged"],       # f32, ragged last chunk
    "2.7b-small": SMALL["2.7b-small"],         # bf16, resident scan, T % 4 != 0
    "2.7b-even": config_by_name("mamba2-2.7b").with_shape(batch=2, seqlen=3 * 256 + 64, nheads=20),
}


@pytest.mark.parametrize("path", ["default", "three"])
@pytest.mark.parametrize("name", sorted(DT_LAYOUT))
def test_dt_head_major_layout(name, path):
    """dt given [batch, nheads, seqlen] (MAMBA2_SSD_DT_HEAD_MAJOR) gives
    bit-identical results to the token-major call, and matches the oracle."""
    cfg = DT_LAYOUT[name]
    pf = 0
    if path == "three":
        if cfg.io != "bf16":
            pytest.skip("the THREE sequence takes bf16 only")
        pf = ssd.PATH_THREE
    log(f"[dt layout] {name} path={path} {cfg}")
    inp = generate(cfg)
    dev = to_device(inp, cfg.io)
    y0, f0 = run(dev, cfg.chunk, path=pf)
    dt_hm = dev["dt"].transpose(1, 2).contiguous()
    y1, f1 = ssd.ssd_fwd(dev["x"], dt_hm, dev["A"], dev["B"], dev["C"], dev["D"], cfg.chunk,
                         dev["init_state"], dt_head_major=True, path=pf)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1), "y differs between the dt layouts"
    assert torch.equal(f0, f1), "final_state differs between the dt layouts"
    yr, fr = oracle_all(inp, cfg)
    check_close(host(y1), yr, cfg.io, "y")
    check_close(host(f1), fr, cfg.io, "final_state")
