"""The C ABI on the host: symbols, validation and workspace arithmetic.

Nothing here launches a kernel; pointers passed to check_args are arbitrary
integers (the library compares them, never dereferences them).
"""
import ctypes
import os
import re
import subprocess

import pytest

import state_space_sequence_ssd_amd as ssd
from state_space_sequence_ssd_amd import BF16, F32, Dims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mamba2_ssd.h")

OK, NULLP, BAD_DIM, GROUPS, CHUNK, UNSUP, WS, ALIAS = 0, -1, -2, -3, -4, -5, -6, -7
ALIGN = -9


HEADERS = [HEADER, os.path.join(ROOT, "include", "mamba1_s6.h")]


def declared_functions():
    names = set()
    for path in HEADERS:
        txt = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"\b(mamba[12]_(?:ssd|s6)_\w+)\s*\(", txt))
    return sorted(names)


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted([
        "mamba2_ssd_check_args", "mamba2_ssd_fwd", "mamba2_ssd_fwd_timed", "mamba2_ssd_fwd_workspace_bytes",
        "mamba2_ssd_last_hip_error", "mamba2_ssd_status_string", "mamba2_ssd_supported",
        "mamba2_ssd_workspace_layout_query", "mamba2_ssd_step", "mamba2_ssd_step_check_args",
        "mamba2_ssd_step_supported", "mamba2_ssd_fused_state_pass", "mamba2_ssd_fwd_path",
        "mamba2_ssd_fwd_noalloc", "mamba2_ssd_bwd",
        "mamba2_ssd_bwd_check_args", "mamba2_ssd_bwd_workspace_bytes", "mamba1_s6_fwd", "mamba1_s6_check_args",
        "mamba1_s6_supported", "mamba1_s6_workspace_bytes", "mamba1_s6_bwd", "mamba1_s6_bwd_check_args",
        "mamba1_s6_bwd_workspace_bytes"])


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", ssd._lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(ssd._lib.lib, name)
        assert getattr(ssd, name) is not None


def test_python_binding_uses_the_same_names():
    for name in declared_functions():
        assert name in ssd.__all__


HEADLINE = Dims(4, 8192, 80, 64, 128, 1, 256)


def test_workspace_layout_headline():
    """Regions per kernel sequence: FOUR holds the chunk states and hprev,
    THREE only hprev, CHAINED neither but the carried-state slots and the
    sync words; unused regions take no bytes."""
    nc = 32
    gq = 4 * 80 * 8192 * 4                      # one [batch][nheads][Tp] fp32 array
    states = 4 * 80 * nc * 64 * 128 * 4
    four = ssd.workspace_layout(HEADLINE, BF16 | ssd.PATH_FOUR)
    assert four.path == ssd.PATH_FOUR and four.nchunks == nc
    assert (four.gcum_offset, four.dtt_offset, four.wst_offset, four.states_offset) == (0, gq, 2 * gq, 3 * gq)
    assert four.hprev_offset == four.states_offset + states
    assert four.chain_offset == four.sync_offset == four.total_bytes == four.hprev_offset + states
    three = ssd.workspace_layout(HEADLINE, BF16 | ssd.PATH_THREE)
    assert three.path == ssd.PATH_THREE
    assert three.states_offset == three.hprev_offset == 3 * gq
    assert three.total_bytes == three.hprev_offset + states
    for L in (four, three):
        for off in (L.gcum_offset, L.dtt_offset, L.wst_offset, L.states_offset, L.hprev_offset, L.total_bytes):
            assert off % 256 == 0
    auto = ssd.workspace_layout(HEADLINE, BF16)
    assert auto.path == ssd.fwd_path(HEADLINE, BF16)
    assert ssd.workspace_bytes(HEADLINE, BF16) == auto.total_bytes
    assert ssd.workspace_bytes(HEADLINE, F32) == four.total_bytes   # fp32 io: four kernels
    ch = ssd.workspace_layout(HEADLINE, BF16 | ssd.PATH_CHAINED)
    assert ch.path == ssd.PATH_CHAINED
    assert ch.wst_offset == ch.states_offset == ch.hprev_offset == ch.chain_offset == 2 * gq   # no w, S, hprev
    assert ch.sync_offset == ch.chain_offset + 4 * 80 * 64 * 128 * 4
    assert ch.total_bytes == ch.sync_offset + ((4 * 80 + 64) * 4 + 255) // 256 * 256
    assert ch.total_bytes <= ssd.NOALLOC_MAX_WORKSPACE     # the headline fits the no-allocation entry point


def test_path_field():
    """The kernel-sequence field of io: forcing a sequence that does not take
    the shape is UNSUPPORTED everywhere; FOUR takes every supported shape."""
    for io in (BF16, F32):
        assert ssd.fwd_path(SMALL, io | ssd.PATH_FOUR) == ssd.PATH_FOUR
        assert _check(SMALL, io | ssd.PATH_FOUR) == OK
    assert ssd.fwd_path(HEADLINE, BF16 | ssd.PATH_THREE) == ssd.PATH_THREE
    assert ssd.fwd_path(HEADLINE, F32) == ssd.PATH_FOUR
    for d, io in ((HEADLINE, F32 | ssd.PATH_THREE),                                   # fp32
                  (Dims(2, 300, 8, 64, 64, 2, 128), BF16 | ssd.PATH_THREE),          # dstate 64, chunk 128
                  (Dims(4, 8192, 80, 128, 64, 1, 256), BF16 | ssd.PATH_THREE)):      # dstate 64, headdim 128
        assert _check(d, io) == UNSUP
        with pytest.raises(ssd.SsdError):
            ssd.fwd_path(d, io)
        assert ssd.workspace_bytes(d, io) == 0
    assert ssd.fwd_path(HEADLINE, BF16 | ssd.PATH_CHAINED) == ssd.PATH_CHAINED
    assert ssd.fwd_path(Dims(1, 65536, 80, 64, 64, 1, 256), BF16 | ssd.PATH_CHAINED) == ssd.PATH_CHAINED
    for d, io in ((HEADLINE, F32), (Dims(4, 8192, 80, 128, 128, 1, 256), BF16),
                  (Dims(4, 8192, 80, 64, 256, 1, 256), BF16), (Dims(4, 8192, 80, 64, 128, 1, 128), BF16)):
        assert _check(d, io | ssd.PATH_CHAINED) == UNSUP    # fp32; headdim 128; dstate 256; chunk 128
    assert ssd.fwd_path(Dims(8, 2048, 24, 64, 128, 1, 256), BF16 | ssd.PATH_FOUR) == ssd.PATH_FOUR


def test_alignment():
    """x, B, C, y, init, final on 16 bytes; dt, A, D on 4; workspace on 256."""
    p, _ = _ptrs(SMALL, BF16)
    for name, off in (("x", 2), ("x", 8), ("B", 8), ("C", 4), ("y", 2), ("init", 8), ("fin", 4), ("dt", 2),
                      ("A", 1), ("D", 2), ("ws", 16)):
        assert _check(SMALL, BF16, **{name: p[name] + off}) == ALIGN, name
    assert _check(SMALL, BF16, ws=p["ws"] + 256) == OK
    assert _check(SMALL, BF16, dt=p["dt"] + 4) == OK


def test_workspace_layout_ragged_pads_to_chunks():
    d = Dims(2, 1000, 8, 64, 64, 2, 128)
    L = ssd.workspace_layout(d, F32)
    assert L.nchunks == 8
    assert L.dtt_offset == ((2 * 8 * 1024 * 4 + 255) // 256) * 256


def test_supported_table():
    for P in (64, 128):
        for N in (64, 128, 256):
            for Q in (64, 128, 256):
                for io in (F32, BF16):
                    assert ssd.supported(P, N, Q, io)
    assert not ssd.supported(32, 128, 256, BF16)
    assert not ssd.supported(64, 96, 256, BF16)
    assert not ssd.supported(64, 128, 32, BF16)
    assert not ssd.supported(64, 128, 256, 7)


def _ptrs(d, io, ws=None):
    """Disjoint fake addresses for every array of a call."""
    e = 2 if io == BF16 else 4
    sizes = {
        "x": d.batch * d.seqlen * d.nheads * d.headdim * e,
        "dt": d.batch * d.seqlen * d.nheads * 4,
        "A": d.nheads * 4, "D": d.nheads * 4,
        "B": d.batch * d.seqlen * d.ngroups * d.dstate * e,
        "C": d.batch * d.seqlen * d.ngroups * d.dstate * e,
        "init": d.batch * d.nheads * d.headdim * d.dstate * 4,
        "y": d.batch * d.seqlen * d.nheads * d.headdim * e,
        "fin": d.batch * d.nheads * d.headdim * d.dstate * 4,
        "ws": ssd.workspace_bytes(d, io) if ws is None else ws,
    }
    p, addr = {}, 1 << 20
    for k, n in sizes.items():
        p[k] = addr
        addr += (n + 4096) // 4096 * 4096 + 4096
    return p, sizes


def _check(d, io, **over):
    p, sizes = _ptrs(d, io)
    p.update({k: v for k, v in over.items() if k != "ws_bytes"})
    return ssd.check_args(d, io, p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["init"], p["y"], p["fin"],
                          p["ws"], over.get("ws_bytes", sizes["ws"]))


SMALL = Dims(2, 300, 8, 64, 128, 2, 128)


def test_valid_call_passes():
    assert _check(SMALL, BF16) == OK
    assert _check(SMALL, F32) == OK
    assert _check(SMALL, BF16, init=0, fin=0) == OK


@pytest.mark.parametrize("field,value,code", [
    ("nheads", 0, BAD_DIM), ("headdim", -1, BAD_DIM), ("batch", -1, BAD_DIM), ("seqlen", -5, BAD_DIM),
    ("ngroups", 3, GROUPS), ("chunk", 100, CHUNK), ("chunk", 32, CHUNK), ("headdim", 96, UNSUP),
    ("dstate", 32, UNSUP), ("seqlen", 1 << 41, BAD_DIM), ("batch", 70000, BAD_DIM),
])
def test_bad_dims(field, value, code):
    d = Dims(*[getattr(SMALL, f) for f, _ in Dims._fields_])
    setattr(d, field, value)
    p, _ = _ptrs(SMALL, BF16)
    assert ssd.check_args(d, BF16, p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["init"], p["y"],
                          p["fin"], p["ws"], 1 << 40) == code
    assert ssd.workspace_bytes(d, BF16) == 0


def test_bad_dtype():
    assert _check(SMALL, 3) == UNSUP


def test_dt_head_major_flag():
    """The dt-layout flag rides in the io argument of every forward entry
    point; it changes nothing that the host checks, and unknown flag bits
    are rejected."""
    hm = ssd.DT_HEAD_MAJOR
    assert hm == 0x100
    for io in (BF16, F32):
        assert _check(SMALL, io | hm) == OK
        assert ssd.workspace_bytes(SMALL, io | hm) == ssd.workspace_bytes(SMALL, io)
        assert ssd.supported(64, 128, 256, io | hm)
    for bad in (BF16 | 0x200, BF16 | 0x10000, F32 | hm | 0x400, 2 | hm):
        assert _check(SMALL, bad) == UNSUP
        assert ssd.workspace_bytes(SMALL, bad) == 0
        assert not ssd.supported(64, 128, 256, bad)
    # the decode step takes no flags
    assert not ssd.step_supported(128, BF16 | hm)


@pytest.mark.parametrize("name", ["x", "dt", "A", "B", "C", "D", "y"])
def test_null_pointers(name):
    assert _check(SMALL, BF16, **{name: 0}) == NULLP


def test_null_dims_struct():
    assert ssd._lib.lib.mamba2_ssd_check_args(None, BF16, 1, 1, 1, 1, 1, 1, 0, 1, 0, 1, 1) == NULLP
    assert ssd._lib.lib.mamba2_ssd_fwd_workspace_bytes(None, BF16) == 0


def test_workspace_errors():
    need = ssd.workspace_bytes(SMALL, BF16)
    assert _check(SMALL, BF16, ws_bytes=need - 1) == WS
    assert _check(SMALL, BF16, ws=0) == WS
    assert _check(SMALL, BF16, ws_bytes=need) == OK


def test_alias_rules():
    p, sizes = _ptrs(SMALL, BF16)
    assert _check(SMALL, BF16, y=p["x"]) == ALIAS
    assert _check(SMALL, BF16, y=p["B"] + 16) == ALIAS
    assert _check(SMALL, BF16, fin=p["init"]) == OK              # in-place state update
    assert _check(SMALL, BF16, fin=p["init"] + 64) == ALIAS       # partial overlap
    assert _check(SMALL, BF16, fin=p["dt"]) == ALIAS
    assert _check(SMALL, BF16, ws=p["y"] + 256) == ALIAS
    assert _check(SMALL, BF16, ws=p["C"]) == ALIAS
    assert _check(SMALL, BF16, C=p["B"]) == OK                     # inputs may overlap each other


def test_empty_problems():
    d0 = Dims(0, 100, 8, 64, 128, 1, 64)
    assert ssd.check_args(d0, BF16, 0, 0, 256, 0, 0, 512, 0, 0, 0, 0, 0) == OK
    dt0 = Dims(2, 0, 8, 64, 128, 1, 64)
    assert ssd.workspace_bytes(dt0, BF16) == 0
    assert ssd.workspace_layout(dt0, BF16).nchunks == 0
    assert ssd.check_args(dt0, BF16, 0, 0, 256, 0, 0, 512, 1 << 30, 0, 1 << 31, 0, 0) == OK
    # fwd with batch 0 returns OK without touching the GPU
    ssd.ssd_fwd_ptr(d0, BF16, 0, 0, 256, 0, 0, 512, 0, 0, 0, 0, 0, 0)


def test_fwd_reports_validation_errors_without_launching():
    with pytest.raises(ssd.SsdError) as e:
        ssd.ssd_fwd_ptr(Dims(1, 64, 3, 64, 64, 2, 64), BF16, 1, 1, 1, 1, 1, 1, 0, 1, 0, 1, 1 << 30, 0)
    assert e.value.status == GROUPS
    assert "multiple" in str(e.value)


def test_noalloc_rejects_oversize_without_a_gpu():
    """The no-allocation entry point checks sizes against its array before
    anything touches the GPU."""
    d = Dims(4, 8192, 80, 64, 128, 1, 256)
    assert ssd.workspace_bytes(d, BF16 | ssd.PATH_FOUR) > ssd.NOALLOC_MAX_WORKSPACE
    lib = ssd._lib.lib
    assert lib.mamba2_ssd_fwd_noalloc(ctypes.byref(d), BF16 | ssd.PATH_FOUR, 256, 256, 256, 256, 256, 256,
                                      0, 1 << 40, 0, 0) == WS
    assert lib.mamba2_ssd_fwd_noalloc(ctypes.byref(Dims(1, 64, 3, 64, 64, 2, 64)), BF16, 1, 1, 1, 1, 1, 1,
                                      0, 1, 0, 0) == GROUPS
    assert lib.mamba2_ssd_fwd_noalloc(None, BF16, 1, 1, 1, 1, 1, 1, 0, 1, 0, 0) == NULLP


def test_status_strings():
    for code in range(-9, 1):
        s = ssd.status_string(code)
        assert s and s != "unknown status"
    assert ssd.status_string(-99) == "unknown status"


# ---------------------------------------------------------------- decode step
STEP = ssd.StepDims(3, 6, 64, 128, 2)


def _step_ptrs(d, io):
    """Disjoint, aligned fake addresses for every step argument."""
    e = 2 if io == BF16 else 4
    sizes = {"x": d.batch * d.nheads * d.headdim * e, "dt": d.batch * d.nheads * 4, "A": d.nheads * 4,
             "D": d.nheads * 4, "B": d.batch * d.ngroups * d.dstate * e, "C": d.batch * d.ngroups * d.dstate * e,
             "state": d.batch * d.nheads * d.headdim * d.dstate * 4, "y": d.batch * d.nheads * d.headdim * e}
    p, base = {}, 1 << 20
    for k, n in sizes.items():
        p[k] = base
        base += (n + 4095) // 4096 * 4096 + 4096
    return p


def _step_check(d, io, **over):
    p = {**_step_ptrs(d, io), **over}
    return ssd.step_check_args(d, io, p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["state"], p["y"])


def test_step_supported_table():
    for io in (F32, BF16):
        for n in (64, 128, 256):
            assert ssd.step_supported(n, io)
        for n in (32, 96, 512):
            assert not ssd.step_supported(n, io)
    assert not ssd.step_supported(128, 7)


def test_step_valid_call_passes():
    assert _step_check(STEP, BF16) == OK
    assert _step_check(STEP, F32) == OK
    assert _step_check(ssd.StepDims(5, 3, 3, 64, 3), F32) == OK      # any headdim


@pytest.mark.parametrize("field,value,code", [("batch", -1, BAD_DIM), ("nheads", 0, BAD_DIM),
                                              ("headdim", 0, BAD_DIM), ("dstate", 96, UNSUP),
                                              ("ngroups", 4, GROUPS), ("ngroups", 0, BAD_DIM),
                                              ("batch", 1 << 30, BAD_DIM)])
def test_step_bad_dims(field, value, code):
    d = ssd.StepDims(STEP.batch, STEP.nheads, STEP.headdim, STEP.dstate, STEP.ngroups)
    setattr(d, field, value)
    p = _step_ptrs(STEP, BF16)
    assert ssd.step_check_args(d, BF16, p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["state"], p["y"]) == code


@pytest.mark.parametrize("name", ["x", "dt", "A", "B", "C", "D", "state", "y"])
def test_step_null_pointers(name):
    assert _step_check(STEP, BF16, **{name: 0}) == NULLP


def test_step_alignment():
    p = _step_ptrs(STEP, BF16)
    assert _step_check(STEP, BF16, state=p["state"] + 8) == ALIGN
    assert _step_check(STEP, BF16, B=p["B"] + 4) == ALIGN
    assert _step_check(STEP, BF16, B=p["B"] + 8) == OK                 # bf16 B/C need 8 bytes
    q = _step_ptrs(STEP, F32)
    assert _step_check(STEP, F32, C=q["C"] + 8) == ALIGN              # fp32 B/C need 16 bytes
    assert _step_check(STEP, F32, x=q["x"] + 2) == ALIGN


def test_step_alias_rules():
    p = _step_ptrs(STEP, BF16)
    assert _step_check(STEP, BF16, y=p["x"]) == ALIAS
    assert _step_check(STEP, BF16, state=p["B"]) == ALIAS
    assert _step_check(STEP, BF16, y=p["state"] + 64) == ALIAS
    assert _step_check(STEP, BF16, state=p["dt"] - 16) == ALIAS


def test_step_empty_and_errors_without_launching():
    assert ssd.step_check_args(ssd.StepDims(0, 4, 64, 128, 1), BF16, 0, 0, 0, 0, 0, 0, 0, 0) == OK
    ssd.ssd_step_ptr(ssd.StepDims(0, 4, 64, 128, 1), BF16, 0, 0, 0, 0, 0, 0, 0, 0)
    with pytest.raises(ssd.SsdError) as e:
        ssd.ssd_step_ptr(ssd.StepDims(1, 3, 64, 128, 2), BF16, 1, 1, 1, 1, 1, 1, 1, 1)
    assert e.value.status == GROUPS
    assert ssd._lib.lib.mamba2_ssd_step_check_args(None, BF16, 1, 1, 1, 1, 1, 1, 1, 1) == NULLP


def test_fused_state_pass_query():
    # the 2.7B-like layer: bf16, headdim 64, 4 x 80 heads x 2 dstate groups
    assert ssd.fused_state_pass(HEADLINE, BF16)
    assert not ssd.fused_state_pass(HEADLINE, F32)                      # fp32 io: four kernels
    assert not ssd.fused_state_pass(Dims(4, 8192, 80, 64, 128, 3, 256), BF16)    # invalid (groups)
    assert not ssd.fused_state_pass(HEADLINE, BF16 | ssd.PATH_FOUR)
    assert ssd.fused_state_pass(Dims(1, 65536, 80, 64, 128, 1, 256), BF16 | ssd.PATH_THREE)
    assert ssd.fused_state_pass(Dims(1, 300, 3, 64, 64, 1, 256), BF16 | ssd.PATH_THREE)
    assert not ssd.fused_state_pass(Dims(1, 300, 3, 64, 64, 1, 128), BF16 | ssd.PATH_THREE)   # dstate 64, chunk 128
    # the row form: dstate 128 or 256, headdim 64 or 128, any chunk
    assert ssd.fused_state_pass(Dims(1, 300, 3, 128, 256, 1, 128), BF16 | ssd.PATH_THREE)
    assert ssd.fused_state_pass(Dims(1, 300, 3, 64, 128, 1, 64), BF16 | ssd.PATH_THREE)
    if ssd.fwd_path(HEADLINE, BF16) != ssd.PATH_CHAINED:
        # without the chained kernel the size rule decides
        assert ssd.fused_state_pass(Dims(4, 8192, 80, 128, 128, 1, 256), BF16)      # 320 row-form walks
        assert ssd.fused_state_pass(Dims(8, 2048, 24, 64, 128, 1, 256), BF16)       # 192 row-form walks
        assert ssd.fused_state_pass(Dims(2, 16384, 64, 128, 256, 8, 128), BF16)     # 256 row-form walks
        assert not ssd.fused_state_pass(Dims(1, 65536, 80, 64, 128, 1, 256), BF16)  # 80 walks: four kernels
        assert not ssd.fused_state_pass(Dims(4, 16384, 8, 64, 128, 1, 128), BF16)   # 32 walks
        assert not ssd.fused_state_pass(Dims(1, 65536, 80, 64, 64, 1, 256), BF16)   # dstate 64: 160 walks
        assert not ssd.fused_state_pass(Dims(4, 0, 80, 64, 128, 1, 256), BF16)      # no chunks


# ------------------------------------------------------------- backward pass

BWD_SMALL = Dims(2, 300, 8, 64, 128, 2, 128)


def _bwd_ptrs(d, io):
    """Disjoint fake addresses for every argument of mamba2_ssd_bwd."""
    e = 2 if io == BF16 else 4
    nx = d.batch * d.seqlen * d.nheads * d.headdim
    nbc = d.batch * d.seqlen * d.ngroups * d.dstate
    nst = d.batch * d.nheads * d.headdim * d.dstate
    sizes = [("x", nx * e), ("dt", d.batch * d.seqlen * d.nheads * 4), ("A", d.nheads * 4), ("B", nbc * e),
             ("C", nbc * e), ("D", d.nheads * 4), ("init", nst * 4), ("dy", nx * e), ("dfinal", nst * 4),
             ("dx", nx * 4), ("ddt", d.batch * d.seqlen * d.nheads * 4), ("dA", d.nheads * 4), ("dB", nbc * 4),
             ("dC", nbc * 4), ("dD", d.nheads * 4), ("dinit", nst * 4),
             ("ws", max(ssd.bwd_workspace_bytes(d, io), 1))]
    p, addr = {}, 1 << 40
    for name, n in sizes:
        p[name] = addr
        addr += (n + 4095) // 4096 * 4096 + 4096
    return p


def _bwd_check(d, io, **over):
    p = _bwd_ptrs(d, io)
    p.update(over)
    ws_bytes = over.get("ws_bytes", ssd.bwd_workspace_bytes(d, io))
    return ssd.bwd_check_args(d, io, p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["init"], p["dy"],
                              p["dfinal"], p["dx"], p["ddt"], p["dA"], p["dB"], p["dC"], p["dD"], p["dinit"],
                              p["ws"], ws_bytes)


def test_bwd_workspace_and_valid_call():
    for io in (BF16, F32):
        assert ssd.bwd_workspace_bytes(BWD_SMALL, io) > 0
        assert _bwd_check(BWD_SMALL, io) == OK
        assert _bwd_check(BWD_SMALL, io, init=0, dfinal=0, dinit=0) == OK
    # the headline layer: fp32 io keeps padded copies and per-head Q x Q
    # blocks (about 9.9 GB); the bf16 fused path needs only these arrays
    assert 9.5e9 < ssd.bwd_workspace_bytes(HEADLINE, F32) < 10.5e9
    bt, T, H, P, N, G, Q = 4, 8192, 80, 64, 128, 1, 256
    nc, Tp = T // Q, T
    nseg = 2   # (b, k, g) items = 128: two head segments make 256 workgroups
    floats = ([bt * H * Tp] * 4 + [bt * Tp * G * N] * 2 + [bt * H * nc * P * N] * 3 + [bt * nc * G * Q * Q]
              + [bt * nc * G * nseg * Q * Q] + [bt * H * nc * P * N] * 2 + [bt * Tp * H * P]
              + [bt * Tp * G * N] * 2 + [bt * H * Tp] * 3 + [bt * H * nc] * 2)
    assert ssd.bwd_workspace_bytes(HEADLINE, BF16) == sum((4 * f + 255) // 256 * 256 for f in floats)


def test_bwd_rejects_bad_calls():
    assert _bwd_check(BWD_SMALL, BF16 | ssd.DT_HEAD_MAJOR) == UNSUP
    assert ssd.bwd_workspace_bytes(BWD_SMALL, BF16 | ssd.DT_HEAD_MAJOR) == 0
    for name in ("x", "dt", "A", "B", "C", "D", "dy", "dx", "ddt", "dA", "dB", "dC", "dD"):
        assert _bwd_check(BWD_SMALL, BF16, **{name: 0}) == NULLP, name
    assert _bwd_check(BWD_SMALL, BF16, ws=0) == WS
    # the workspace's regions are read in 16-byte pieces from 256-byte offsets
    assert _bwd_check(BWD_SMALL, BF16, ws=_bwd_ptrs(BWD_SMALL, BF16)["ws"] + 16) == ALIGN
    assert _bwd_check(BWD_SMALL, BF16, ws_bytes=ssd.bwd_workspace_bytes(BWD_SMALL, BF16) - 1) == WS
    p = _bwd_ptrs(BWD_SMALL, BF16)
    # an output on an input, on another output, or on the workspace
    assert _bwd_check(BWD_SMALL, BF16, dx=p["x"]) == ALIAS
    assert _bwd_check(BWD_SMALL, BF16, dB=p["dC"]) == ALIAS
    assert _bwd_check(BWD_SMALL, BF16, dinit=p["ws"]) == ALIAS
    assert _bwd_check(BWD_SMALL, BF16, dinit=p["init"]) == ALIAS
    # batch * nchunks * nheads beyond one grid dimension
    big = Dims(64, 65536, 80, 64, 128, 1, 256)
    assert ssd.bwd_workspace_bytes(big, BF16) == 0


def test_bwd_fails_without_launching():
    p = _bwd_ptrs(BWD_SMALL, BF16)
    args = [p[k] for k in ("x", "dt", "A", "B", "C", "D", "init", "dy", "dfinal", "dx", "ddt", "dA", "dB", "dC",
                           "dD", "dinit", "ws")]
    args[0] = 0
    with pytest.raises(ssd.SsdError):
        ssd.ssd_bwd_ptr(BWD_SMALL, BF16, *args, ssd.bwd_workspace_bytes(BWD_SMALL, BF16))


# ----------------------------------------------------- selective scan (S6)

S6_SMALL = ssd.S6Dims(2, 300, 96, 16)


def _s6_ptrs(d):
    sizes = [("x", d.batch * d.channels * d.seqlen * 4), ("delta", d.batch * d.channels * d.seqlen * 4),
             ("A", d.channels * d.dstate * 4), ("B", d.batch * d.dstate * d.seqlen * 4),
             ("C", d.batch * d.dstate * d.seqlen * 4), ("h0", d.batch * d.channels * d.dstate * 4),
             ("y", d.batch * d.channels * d.seqlen * 4), ("hT", d.batch * d.channels * d.dstate * 4),
             ("ws", max(ssd.s6_workspace_bytes(d), 1))]
    p, addr = {}, 1 << 40
    for name, n in sizes:
        p[name] = addr
        addr += (n + 4095) // 4096 * 4096 + 4096
    return p


def _s6_check(d, **over):
    p = _s6_ptrs(d)
    p.update(over)
    wsb = over.get("ws_bytes", ssd.s6_workspace_bytes(d))
    return ssd.s6_check_args(d, p["x"], p["delta"], p["A"], p["B"], p["C"], p["h0"], p["y"], p["hT"], p["ws"], wsb)


def test_s6_supported_and_workspace():
    assert [n for n in range(1, 33) if ssd.s6_supported(n)] == [1, 2, 4, 8, 16]
    # per (b, chunk, d): the chunk's end state from zero and its inclusive end
    # state (N floats each) and its delta sum; then 64 sync words and one
    # flag per (b, chunk, block of 256 channels)
    nc = (300 + 63) // 64
    want = sum((n * 4 + 255) // 256 * 256
               for n in (2 * 96 * nc * 16, 2 * 96 * nc, 2 * 96 * nc * 16, 64 + nc * 2 * 1))
    assert ssd.s6_workspace_bytes(S6_SMALL) == want


def test_s6_validation():
    assert _s6_check(S6_SMALL) == OK
    assert _s6_check(S6_SMALL, h0=0, hT=0) == OK
    for name in ("x", "delta", "A", "B", "C", "y"):
        assert _s6_check(S6_SMALL, **{name: 0}) == NULLP, name
    p = _s6_ptrs(S6_SMALL)
    assert _s6_check(S6_SMALL, y=p["x"]) == ALIAS
    assert _s6_check(S6_SMALL, hT=p["h0"]) == OK          # in place
    assert _s6_check(S6_SMALL, hT=p["h0"] + 4) == ALIAS   # partial overlap
    assert _s6_check(S6_SMALL, ws=0) == WS
    # float arrays at 4 bytes, the workspace at 256 bytes
    for name in ("x", "delta", "A", "B", "C", "h0", "y", "hT"):
        assert _s6_check(S6_SMALL, **{name: p[name] + 2}) == ALIGN, name
    assert _s6_check(S6_SMALL, ws=p["ws"] + 16) == ALIGN
    assert _s6_check(S6_SMALL, x=p["x"] + 4, y=p["y"] + 8) == OK   # 4-byte offsets take the 4-byte loads
    bad = ssd.S6Dims(2, 300, 96, 12)
    assert ssd.s6_workspace_bytes(bad) == 0 and _s6_check(bad) == UNSUP
    assert ssd.s6_workspace_bytes(ssd.S6Dims(70000, 10, 4, 4)) == 0
    assert ssd.s6_workspace_bytes(ssd.S6Dims(1, 64 * 65536, 4, 4)) == 0
    assert _s6_check(ssd.S6Dims(0, 300, 96, 16), x=0, delta=0, B=0, C=0, y=0, ws=0) == OK


def _s6_bwd_ptrs(d):
    bt, L, D, N = d.batch, d.seqlen, d.channels, d.dstate
    sizes = {"x": bt * D * L, "delta": bt * D * L, "A": D * N, "B": bt * N * L, "C": bt * N * L,
             "h0": bt * D * N, "dy": bt * D * L, "dhT": bt * D * N, "dx": bt * D * L, "ddelta": bt * D * L,
             "dA": D * N, "dB": bt * N * L, "dC": bt * N * L, "dh0": bt * D * N}
    p, base = {}, 1 << 40
    for k, n in sizes.items():
        p[k] = base
        base += (4 * n + 4095) // 4096 * 4096 + 4096
    p["ws"] = base
    return p


def _s6_bwd_check(d, **over):
    p = _s6_bwd_ptrs(d)
    p.update(over)
    ws_bytes = over.get("ws_bytes", ssd.s6_bwd_workspace_bytes(d))
    return ssd.s6_bwd_check_args(d, p["x"], p["delta"], p["A"], p["B"], p["C"], p["h0"], p["dy"], p["dhT"], p["dx"],
                                 p["ddelta"], p["dA"], p["dB"], p["dC"], p["dh0"], p["ws"], ws_bytes)


def test_s6_bwd_workspace_and_validation():
    # the forward's workspace, then per (b, chunk, d): the chunk's outgoing
    # adjoint, its delta sum, its entering adjoint and its dA part; per
    # (b, block of 64 channels): the dB and dC parts
    nc, ncb = (300 + 63) // 64, 2
    fwd = ssd.s6_workspace_bytes(ssd.S6Dims(2, 300, 96, 4))
    d4 = ssd.S6Dims(2, 300, 96, 4)
    want = fwd + sum((n * 4 + 255) // 256 * 256 for n in (2 * nc * 96 * 4, 2 * nc * 96, 2 * nc * 96 * 4,
                                                          2 * nc * 96 * 4, 2 * ncb * 4 * 300, 2 * ncb * 4 * 300))
    assert ssd.s6_bwd_workspace_bytes(d4) == want
    assert _s6_bwd_check(d4) == OK
    assert _s6_bwd_check(d4, h0=0, dhT=0, dh0=0) == OK
    for name in ("x", "delta", "A", "B", "C", "dy", "dx", "ddelta", "dA", "dB", "dC"):
        assert _s6_bwd_check(d4, **{name: 0}) == NULLP, name
    p = _s6_bwd_ptrs(d4)
    assert _s6_bwd_check(d4, dx=p["x"]) == ALIAS
    assert _s6_bwd_check(d4, dB=p["dC"]) == ALIAS
    assert _s6_bwd_check(d4, dh0=p["h0"]) == ALIAS
    assert _s6_bwd_check(d4, ws=0) == WS
    for name in ("x", "dy", "dhT", "dx", "dA", "dB", "dh0"):
        assert _s6_bwd_check(d4, **{name: p[name] + 2}) == ALIGN, name
    assert _s6_bwd_check(d4, ws=p["ws"] + 64) == ALIGN
    assert _s6_bwd_check(d4, dB=p["dB"] + 4, dC=p["dC"] + 12) == OK
    # every dstate of the forward scan has a backward pass (dstate 16 in four
    # passes of 4 states); others are unsupported
    assert ssd.s6_bwd_workspace_bytes(ssd.S6Dims(2, 300, 96, 16)) > 0
    assert _s6_bwd_check(ssd.S6Dims(2, 300, 96, 16)) == OK
    assert _s6_bwd_check(ssd.S6Dims(2, 300, 96, 12)) == UNSUP
    # empty batch: only A and dA are needed
    e = ssd.S6Dims(0, 300, 96, 4)
    assert _s6_bwd_check(e, x=0, delta=0, B=0, C=0, dy=0, dx=0, ddelta=0, dB=0, dC=0, ws=0) == OK
