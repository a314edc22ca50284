"""ctypes loader and prototypes for libmamba2_ssd.so (see include/mamba2_ssd.h)."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmamba2_ssd.so")

F32 = 0
BF16 = 1
DT_HEAD_MAJOR = 0x100   # OR-ed into io: dt given as [batch, nheads, seqlen]
# kernel sequence, a field OR-ed into io (see include/mamba2_ssd.h)
PATH_AUTO, PATH_FOUR, PATH_THREE, PATH_CHAINED = 0x0000, 0x1000, 0x2000, 0x3000
PATH_NAMES = {PATH_FOUR: "four", PATH_THREE: "three", PATH_CHAINED: "chained"}
NOALLOC_MAX_WORKSPACE = 64 << 20   # MAMBA2_SSD_NOALLOC_MAX_WORKSPACE

STATUS = {
    0: "OK",
    -1: "ERR_NULL_POINTER",
    -2: "ERR_BAD_DIM",
    -3: "ERR_GROUPS",
    -4: "ERR_CHUNK",
    -5: "ERR_UNSUPPORTED",
    -6: "ERR_WORKSPACE",
    -7: "ERR_ALIAS",
    -8: "ERR_HIP",
    -9: "ERR_ALIGN",
}


class Dims(ctypes.Structure):
    """mamba2_ssd_dims"""
    _fields_ = [(n, ctypes.c_int64) for n in
                ("batch", "seqlen", "nheads", "headdim", "dstate", "ngroups", "chunk")]


class StepDims(ctypes.Structure):
    """mamba2_ssd_step_dims"""
    _fields_ = [(n, ctypes.c_int64) for n in ("batch", "nheads", "headdim", "dstate", "ngroups")]


class S6Dims(ctypes.Structure):
    """mamba1_s6_dims"""
    _fields_ = [(n, ctypes.c_int64) for n in ("batch", "seqlen", "channels", "dstate")]


class WorkspaceLayout(ctypes.Structure):
    """mamba2_ssd_workspace_layout"""
    _fields_ = [("total_bytes", ctypes.c_size_t), ("gcum_offset", ctypes.c_size_t),
                ("dtt_offset", ctypes.c_size_t), ("wst_offset", ctypes.c_size_t),
                ("states_offset", ctypes.c_size_t), ("hprev_offset", ctypes.c_size_t),
                ("chain_offset", ctypes.c_size_t), ("sync_offset", ctypes.c_size_t),
                ("nchunks", ctypes.c_int64), ("path", ctypes.c_int32)]


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            return sorted({l.split()[-1] for l in f if "libamdhip64" in l})
    except OSError:
        return []


def _load():
    # One process must hold one HIP runtime. PyTorch ships its own
    # libamdhip64 whose SONAME matches ROCm's, so importing torch first makes
    # the dynamic loader bind this library to that already-loaded runtime
    # instead of mapping a second one (two runtimes cannot share the device).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python state_space_sequence_ssd_amd/build.py`. "
            "There is no CPU fallback for the SSD forward pass.")
    L = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are mapped in this process (" + ", ".join(runtimes) +
                          "); import torch before loading libmamba2_ssd.so")
    vp, fp, i64, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    dims_p = ctypes.POINTER(Dims)
    L.mamba2_ssd_supported.argtypes = [i64, i64, i64, ctypes.c_int]
    L.mamba2_ssd_supported.restype = ctypes.c_int
    L.mamba2_ssd_workspace_layout_query.argtypes = [dims_p, ctypes.c_int, ctypes.POINTER(WorkspaceLayout)]
    L.mamba2_ssd_workspace_layout_query.restype = ctypes.c_int
    L.mamba2_ssd_fwd_workspace_bytes.argtypes = [dims_p, ctypes.c_int]
    L.mamba2_ssd_fwd_workspace_bytes.restype = sz
    L.mamba2_ssd_check_args.argtypes = [dims_p, ctypes.c_int, vp, fp, fp, vp, vp, fp, fp, vp, fp, vp, sz]
    L.mamba2_ssd_check_args.restype = ctypes.c_int
    L.mamba2_ssd_fwd.argtypes = [dims_p, ctypes.c_int, vp, fp, fp, vp, vp, fp, fp, vp, fp, vp, sz, vp]
    L.mamba2_ssd_fwd.restype = ctypes.c_int
    L.mamba2_ssd_fwd_timed.argtypes = [dims_p, ctypes.c_int, vp, fp, fp, vp, vp, fp, fp, vp, fp, vp, sz, vp,
                                       ctypes.POINTER(ctypes.c_void_p)]
    L.mamba2_ssd_fwd_timed.restype = ctypes.c_int
    L.mamba2_ssd_fwd_noalloc.argtypes = [dims_p, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.mamba2_ssd_fwd_noalloc.restype = ctypes.c_int
    L.mamba2_ssd_fwd_path.argtypes = [dims_p, ctypes.c_int]
    L.mamba2_ssd_fwd_path.restype = ctypes.c_int
    L.mamba2_ssd_fused_state_pass.argtypes = [dims_p, ctypes.c_int]
    L.mamba2_ssd_fused_state_pass.restype = ctypes.c_int
    L.mamba2_ssd_bwd_workspace_bytes.argtypes = [dims_p, ctypes.c_int]
    L.mamba2_ssd_bwd_workspace_bytes.restype = sz
    L.mamba2_ssd_bwd_check_args.argtypes = [dims_p, ctypes.c_int, vp, fp, fp, vp, vp, fp, fp, vp, fp,
                                            fp, fp, fp, fp, fp, fp, fp, vp, sz]
    L.mamba2_ssd_bwd_check_args.restype = ctypes.c_int
    L.mamba2_ssd_bwd.argtypes = [dims_p, ctypes.c_int, vp, fp, fp, vp, vp, fp, fp, vp, fp,
                                 fp, fp, fp, fp, fp, fp, fp, vp, sz, vp]
    L.mamba2_ssd_bwd.restype = ctypes.c_int
    s6_p = ctypes.POINTER(S6Dims)
    L.mamba1_s6_supported.argtypes = [i64]
    L.mamba1_s6_supported.restype = ctypes.c_int
    L.mamba1_s6_workspace_bytes.argtypes = [s6_p]
    L.mamba1_s6_workspace_bytes.restype = sz
    L.mamba1_s6_check_args.argtypes = [s6_p, fp, fp, fp, fp, fp, fp, fp, fp, vp, sz]
    L.mamba1_s6_check_args.restype = ctypes.c_int
    L.mamba1_s6_fwd.argtypes = [s6_p, fp, fp, fp, fp, fp, fp, fp, fp, vp, sz, vp]
    L.mamba1_s6_fwd.restype = ctypes.c_int
    L.mamba1_s6_bwd_workspace_bytes.argtypes = [s6_p]
    L.mamba1_s6_bwd_workspace_bytes.restype = sz
    L.mamba1_s6_bwd_check_args.argtypes = [s6_p] + [fp] * 14 + [vp, sz]
    L.mamba1_s6_bwd_check_args.restype = ctypes.c_int
    L.mamba1_s6_bwd.argtypes = [s6_p] + [fp] * 14 + [vp, sz, vp]
    L.mamba1_s6_bwd.restype = ctypes.c_int
    step_p = ctypes.POINTER(StepDims)
    L.mamba2_ssd_step_supported.argtypes = [i64, ctypes.c_int]
    L.mamba2_ssd_step_supported.restype = ctypes.c_int
    L.mamba2_ssd_step_check_args.argtypes = [step_p, ctypes.c_int, vp, fp, fp, vp, vp, fp, fp, vp]
    L.mamba2_ssd_step_check_args.restype = ctypes.c_int
    L.mamba2_ssd_step.argtypes = [step_p, ctypes.c_int, vp, fp, fp, vp, vp, fp, fp, vp, vp]
    L.mamba2_ssd_step.restype = ctypes.c_int
    L.mamba2_ssd_status_string.argtypes = [ctypes.c_int]
    L.mamba2_ssd_status_string.restype = ctypes.c_char_p
    L.mamba2_ssd_last_hip_error.argtypes = []
    L.mamba2_ssd_last_hip_error.restype = ctypes.c_char_p
    return L


lib = _load()


def status_string(status: int) -> str:
    return lib.mamba2_ssd_status_string(status).decode()


class SsdError(RuntimeError):
    """A nonzero status from the library."""

    def __init__(self, status: int, detail: str = ""):
        self.status = status
        msg = f"mamba2_ssd: {STATUS.get(status, status)} ({status_string(status)})"
        if detail:
            msg += f": {detail}"
        super().__init__(msg)
