"""Mamba-2 chunked SSD forward pass for AMD MI355X (gfx950).

A thin binding of ``libmamba2_ssd.so`` (C ABI in ``include/mamba2_ssd.h``).
Every step of the forward pass runs in the library's HIP kernels; this module
only marshals arguments. PyTorch provides device memory and the current
stream. Importing raises if the library has not been built
(``python state_space_sequence_ssd_amd/build.py``); there is no fallback.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

from ._lib import (BF16, DT_HEAD_MAJOR, F32, NOALLOC_MAX_WORKSPACE, PATH_AUTO, PATH_CHAINED, PATH_FOUR, PATH_NAMES, PATH_THREE, STATUS,
                   Dims, S6Dims, SsdError, StepDims, WorkspaceLayout, lib, status_string)

__all__ = ["ssd_fwd", "ssd_fwd_ptr", "supported", "workspace_bytes", "workspace_layout", "check_args",
           "Dims", "WorkspaceLayout", "SsdError", "F32", "BF16", "DT_HEAD_MAJOR", "STATUS", "status_string",
           "ssd_fwd_timed_ptr", "mamba2_ssd_fwd", "mamba2_ssd_fwd_timed", "mamba2_ssd_check_args",
           "mamba2_ssd_supported",
           "mamba2_ssd_fwd_workspace_bytes", "mamba2_ssd_workspace_layout_query",
           "mamba2_ssd_status_string", "mamba2_ssd_last_hip_error",
           "ssd_step", "ssd_step_ptr", "step_supported", "step_check_args", "StepDims",
           "mamba2_ssd_step", "mamba2_ssd_step_check_args", "mamba2_ssd_step_supported",
           "mamba2_ssd_fused_state_pass", "fused_state_pass", "mamba2_ssd_fwd_path", "fwd_path",
           "PATH_AUTO", "PATH_FOUR", "PATH_THREE", "PATH_CHAINED", "PATH_NAMES",
           "mamba2_ssd_fwd_noalloc", "ssd_fwd_noalloc_ptr", "NOALLOC_MAX_WORKSPACE",
           "ssd_bwd", "ssd_bwd_ptr", "bwd_workspace_bytes", "bwd_check_args",
           "mamba2_ssd_bwd", "mamba2_ssd_bwd_check_args", "mamba2_ssd_bwd_workspace_bytes",
           "S6Dims", "s6_fwd", "s6_fwd_ptr", "s6_supported", "s6_workspace_bytes", "s6_check_args",
           "mamba1_s6_fwd", "mamba1_s6_check_args", "mamba1_s6_supported", "mamba1_s6_workspace_bytes",
           "S6_GRAD_NAMES", "s6_bwd", "s6_bwd_ptr", "s6_bwd_workspace_bytes", "s6_bwd_check_args",
           "mamba1_s6_bwd", "mamba1_s6_bwd_check_args", "mamba1_s6_bwd_workspace_bytes"]

# The C entry points under their own names (ctypes functions with prototypes).
mamba2_ssd_fwd = lib.mamba2_ssd_fwd
mamba2_ssd_fwd_timed = lib.mamba2_ssd_fwd_timed
mamba2_ssd_check_args = lib.mamba2_ssd_check_args
mamba2_ssd_supported = lib.mamba2_ssd_supported
mamba2_ssd_fwd_workspace_bytes = lib.mamba2_ssd_fwd_workspace_bytes
mamba2_ssd_workspace_layout_query = lib.mamba2_ssd_workspace_layout_query
mamba2_ssd_status_string = lib.mamba2_ssd_status_string
mamba2_ssd_last_hip_error = lib.mamba2_ssd_last_hip_error
mamba2_ssd_fused_state_pass = lib.mamba2_ssd_fused_state_pass
mamba2_ssd_fwd_path = lib.mamba2_ssd_fwd_path
mamba2_ssd_fwd_noalloc = lib.mamba2_ssd_fwd_noalloc
mamba2_ssd_step = lib.mamba2_ssd_step
mamba2_ssd_step_check_args = lib.mamba2_ssd_step_check_args
mamba2_ssd_step_supported = lib.mamba2_ssd_step_supported
mamba2_ssd_bwd = lib.mamba2_ssd_bwd
mamba1_s6_fwd = lib.mamba1_s6_fwd
mamba1_s6_check_args = lib.mamba1_s6_check_args
mamba1_s6_supported = lib.mamba1_s6_supported
mamba1_s6_workspace_bytes = lib.mamba1_s6_workspace_bytes
mamba1_s6_bwd = lib.mamba1_s6_bwd
mamba1_s6_bwd_check_args = lib.mamba1_s6_bwd_check_args
mamba1_s6_bwd_workspace_bytes = lib.mamba1_s6_bwd_workspace_bytes
mamba2_ssd_bwd_check_args = lib.mamba2_ssd_bwd_check_args
mamba2_ssd_bwd_workspace_bytes = lib.mamba2_ssd_bwd_workspace_bytes


def _dims(d) -> Dims:
    if isinstance(d, Dims):
        return d
    if isinstance(d, dict):
        return Dims(**d)
    return Dims(*d)


def supported(headdim: int, dstate: int, chunk: int, io: int) -> bool:
    return bool(lib.mamba2_ssd_supported(headdim, dstate, chunk, io))


def workspace_layout(dims, io: int) -> WorkspaceLayout:
    out = WorkspaceLayout()
    st = lib.mamba2_ssd_workspace_layout_query(ctypes.byref(_dims(dims)), io, ctypes.byref(out))
    if st != 0:
        raise SsdError(st)
    return out


def fused_state_pass(dims, io: int) -> bool:
    """Whether a forward call with these sizes computes the chunk states inside
    the state pass (then the workspace's states region is not written)."""
    return bool(lib.mamba2_ssd_fused_state_pass(ctypes.byref(_dims(dims)), io))


def fwd_path(dims, io: int) -> int:
    """The kernel sequence (PATH_FOUR, PATH_THREE or PATH_CHAINED) a forward
    call with these sizes and io value (including its path field) takes;
    raises SsdError when the arguments are invalid or the forced sequence does
    not support the shape."""
    st = int(lib.mamba2_ssd_fwd_path(ctypes.byref(_dims(dims)), io))
    if st < 0:
        raise SsdError(st)
    return st


def workspace_bytes(dims, io: int) -> int:
    return int(lib.mamba2_ssd_fwd_workspace_bytes(ctypes.byref(_dims(dims)), io))


def check_args(dims, io, x, dt, A, B, C, D, init_state, y, final_state, workspace, ws_bytes) -> int:
    """Host-only validation on raw integer addresses (0 for NULL)."""
    return int(lib.mamba2_ssd_check_args(ctypes.byref(_dims(dims)), io, x, dt, A, B, C, D,
                                         init_state, y, final_state, workspace, ws_bytes))


def ssd_fwd_ptr(dims, io, x, dt, A, B, C, D, init_state, y, final_state, workspace, ws_bytes,
                stream: int = 0) -> None:
    """mamba2_ssd_fwd on raw device addresses; raises SsdError on a nonzero status."""
    st = lib.mamba2_ssd_fwd(ctypes.byref(_dims(dims)), io, x, dt, A, B, C, D, init_state, y,
                            final_state, workspace, ws_bytes, stream)
    if st != 0:
        raise SsdError(st, lib.mamba2_ssd_last_hip_error().decode())


def ssd_fwd_noalloc_ptr(dims, io, x, dt, A, B, C, D, init_state, y, final_state, stream: int = 0) -> None:
    """mamba2_ssd_fwd_noalloc on raw device addresses (the workspace is the
    library's own device array); raises SsdError on a nonzero status."""
    st = lib.mamba2_ssd_fwd_noalloc(ctypes.byref(_dims(dims)), io, x, dt, A, B, C, D, init_state, y,
                                    final_state, stream)
    if st != 0:
        raise SsdError(st, lib.mamba2_ssd_last_hip_error().decode())


def ssd_fwd_timed_ptr(dims, io, x, dt, A, B, C, D, init_state, y, final_state, workspace, ws_bytes,
                      stream: int, events) -> None:
    """mamba2_ssd_fwd_timed on raw addresses; ``events`` holds 5 hipEvent_t handles."""
    arr = (ctypes.c_void_p * 5)(*events)
    st = lib.mamba2_ssd_fwd_timed(ctypes.byref(_dims(dims)), io, x, dt, A, B, C, D, init_state, y,
                                  final_state, workspace, ws_bytes, stream, arr)
    if st != 0:
        raise SsdError(st, lib.mamba2_ssd_last_hip_error().decode())


def ssd_fwd(x, dt, A, B, C, D, chunk: int, init_state=None, *, return_final_state: bool = True,
            y=None, final_state=None, workspace=None,
            dt_head_major: bool = False, path: int = PATH_AUTO) -> Tuple[object, Optional[object]]:
    """Forward pass on torch CUDA tensors (all contiguous, same device).

    x [batch, seqlen, nheads, headdim] and B, C [batch, seqlen, ngroups,
    dstate] share the io dtype (torch.bfloat16 or torch.float32); dt
    [batch, seqlen, nheads] (or [batch, nheads, seqlen] with
    ``dt_head_major``), A and D [nheads] and init_state [batch, nheads,
    headdim, dstate] are float32. Returns ``(y, final_state)``; final_state is
    None when ``return_final_state`` is False. ``y``, ``final_state`` and
    ``workspace`` (a uint8 tensor) may be passed to reuse memory; otherwise
    they are allocated with torch. ``path`` forces a kernel sequence
    (PATH_FOUR, PATH_THREE, PATH_CHAINED; PATH_AUTO lets the library choose).
    Runs on torch's current stream.
    """
    import torch

    if x.dtype == torch.bfloat16:
        io = BF16
    elif x.dtype == torch.float32:
        io = F32
    else:
        raise TypeError(f"x must be bfloat16 or float32, got {x.dtype}")
    for name, t, want in (("B", B, x.dtype), ("C", C, x.dtype), ("dt", dt, torch.float32),
                          ("A", A, torch.float32), ("D", D, torch.float32)):
        if t.dtype != want:
            raise TypeError(f"{name} must be {want}, got {t.dtype}")
    if init_state is not None and init_state.dtype != torch.float32:
        raise TypeError("init_state must be float32")
    tensors = [x, dt, A, B, C, D] + ([init_state] if init_state is not None else [])
    for t in tensors:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dt_shape = (bt, H, T) if dt_head_major else (bt, T, H)
    if tuple(dt.shape) != dt_shape or tuple(B.shape) != (bt, T, G, N) or tuple(C.shape) != (bt, T, G, N) \
            or tuple(A.shape) != (H,) or tuple(D.shape) != (H,):
        raise ValueError("inconsistent shapes")
    if init_state is not None and tuple(init_state.shape) != (bt, H, P, N):
        raise ValueError("init_state must be [batch, nheads, headdim, dstate]")
    dims = Dims(bt, T, H, P, N, G, chunk)
    if dt_head_major:
        io |= DT_HEAD_MAJOR
    io |= path
    if y is None:
        y = torch.empty_like(x)
    if return_final_state and final_state is None:
        final_state = torch.empty((bt, H, P, N), dtype=torch.float32, device=x.device)
    nbytes = workspace_layout(dims, io).total_bytes   # raises SsdError on invalid sizes
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    ptr = lambda t: 0 if t is None else t.data_ptr()
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        ssd_fwd_ptr(dims, io, ptr(x), ptr(dt), ptr(A), ptr(B), ptr(C), ptr(D), ptr(init_state), ptr(y),
                    ptr(final_state) if return_final_state else 0, ptr(workspace), workspace.numel(), stream)
    return y, (final_state if return_final_state else None)


def _step_dims(d) -> StepDims:
    if isinstance(d, StepDims):
        return d
    if isinstance(d, dict):
        return StepDims(**d)
    return StepDims(*d)


def step_supported(dstate: int, io: int) -> bool:
    return bool(lib.mamba2_ssd_step_supported(dstate, io))


def step_check_args(dims, io, x, dt, A, B, C, D, state, y) -> int:
    """Host-only validation of a decode step on raw integer addresses (0 for NULL)."""
    return int(lib.mamba2_ssd_step_check_args(ctypes.byref(_step_dims(dims)), io, x, dt, A, B, C, D, state, y))


def ssd_step_ptr(dims, io, x, dt, A, B, C, D, state, y, stream: int = 0) -> None:
    """mamba2_ssd_step on raw device addresses; raises SsdError on a nonzero status."""
    st = lib.mamba2_ssd_step(ctypes.byref(_step_dims(dims)), io, x, dt, A, B, C, D, state, y, stream)
    if st != 0:
        raise SsdError(st, lib.mamba2_ssd_last_hip_error().decode())


def ssd_step(x, dt, A, B, C, D, state, *, y=None):
    """One decode step on torch CUDA tensors (contiguous, same device).

    x [batch, nheads, headdim] and B, C [batch, ngroups, dstate] share the io
    dtype (torch.bfloat16 or torch.float32); dt [batch, nheads], A and D
    [nheads] and state [batch, nheads, headdim, dstate] are float32. The
    state is updated in place; returns y [batch, nheads, headdim] in the io
    dtype (written into ``y`` when given). Runs on torch's current stream.
    """
    import torch

    if x.dtype == torch.bfloat16:
        io = BF16
    elif x.dtype == torch.float32:
        io = F32
    else:
        raise TypeError(f"x must be bfloat16 or float32, got {x.dtype}")
    for name, t, want in (("B", B, x.dtype), ("C", C, x.dtype), ("dt", dt, torch.float32),
                          ("A", A, torch.float32), ("D", D, torch.float32), ("state", state, torch.float32)):
        if t.dtype != want:
            raise TypeError(f"{name} must be {want}, got {t.dtype}")
    for t in (x, dt, A, B, C, D, state):
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    bt, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    if tuple(dt.shape) != (bt, H) or tuple(B.shape) != (bt, G, N) or tuple(C.shape) != (bt, G, N) \
            or tuple(A.shape) != (H,) or tuple(D.shape) != (H,) or tuple(state.shape) != (bt, H, P, N):
        raise ValueError("inconsistent shapes")
    if y is None:
        y = torch.empty_like(x)
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        ssd_step_ptr(StepDims(bt, H, P, N, G), io, x.data_ptr(), dt.data_ptr(), A.data_ptr(), B.data_ptr(),
                     C.data_ptr(), D.data_ptr(), state.data_ptr(), y.data_ptr(), stream)
    return y


# ------------------------------------------------------------- backward pass

GRAD_NAMES = ("dx", "ddt", "dA", "dB", "dC", "dD", "dinit")


def bwd_workspace_bytes(dims, io: int) -> int:
    return int(lib.mamba2_ssd_bwd_workspace_bytes(ctypes.byref(_dims(dims)), io))


def bwd_check_args(dims, io, x, dt, A, B, C, D, init_state, dy, dfinal, dx, ddt, dA, dB, dC, dD, dinit,
                   workspace, ws_bytes) -> int:
    """Host-only validation of a backward call on raw integer addresses (0 for NULL)."""
    return int(lib.mamba2_ssd_bwd_check_args(ctypes.byref(_dims(dims)), io, x, dt, A, B, C, D, init_state, dy,
                                             dfinal, dx, ddt, dA, dB, dC, dD, dinit, workspace, ws_bytes))


def ssd_bwd_ptr(dims, io, x, dt, A, B, C, D, init_state, dy, dfinal, dx, ddt, dA, dB, dC, dD, dinit,
                workspace, ws_bytes, stream: int = 0) -> None:
    """mamba2_ssd_bwd on raw device addresses; raises SsdError on a nonzero status."""
    st = lib.mamba2_ssd_bwd(ctypes.byref(_dims(dims)), io, x, dt, A, B, C, D, init_state, dy, dfinal, dx, ddt,
                            dA, dB, dC, dD, dinit, workspace, ws_bytes, stream)
    if st != 0:
        raise SsdError(st, lib.mamba2_ssd_last_hip_error().decode())


def ssd_bwd(x, dt, A, B, C, D, dy, chunk: int, init_state=None, dfinal=None, *, workspace=None) -> dict:
    """Gradients of the forward pass on torch CUDA tensors (contiguous, one
    device): ``dy`` like y (the io dtype), ``dfinal`` float32 like the final
    state or None. Returns a dict of float32 tensors named dx, ddt, dA, dB,
    dC, dD and dinit (the initial state's gradient, also when init_state is
    None). Runs on torch's current stream.
    """
    import torch

    io = BF16 if x.dtype == torch.bfloat16 else F32
    if x.dtype not in (torch.bfloat16, torch.float32) or dy.dtype != x.dtype or B.dtype != x.dtype \
            or C.dtype != x.dtype:
        raise TypeError("x, B, C and dy must share the io dtype (bfloat16 or float32)")
    for name, t in (("dt", dt), ("A", A), ("D", D), ("init_state", init_state), ("dfinal", dfinal)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    for t in (x, dt, A, B, C, D, dy, init_state, dfinal):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("all tensors must be contiguous GPU tensors")
    bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if tuple(dy.shape) != tuple(x.shape) or tuple(dt.shape) != (bt, T, H):
        raise ValueError("inconsistent shapes")
    dims = Dims(bt, T, H, P, N, G, chunk)
    f32 = dict(dtype=torch.float32, device=x.device)
    g = {"dx": torch.empty((bt, T, H, P), **f32), "ddt": torch.empty((bt, T, H), **f32),
         "dA": torch.empty((H,), **f32), "dB": torch.empty((bt, T, G, N), **f32),
         "dC": torch.empty((bt, T, G, N), **f32), "dD": torch.empty((H,), **f32),
         "dinit": torch.empty((bt, H, P, N), **f32)}
    nbytes = bwd_workspace_bytes(dims, io)   # 0 for invalid sizes too: the call then reports the status
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    ptr = lambda t: 0 if t is None else t.data_ptr()
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        ssd_bwd_ptr(dims, io, ptr(x), ptr(dt), ptr(A), ptr(B), ptr(C), ptr(D), ptr(init_state), ptr(dy),
                    ptr(dfinal), *[ptr(g[k]) for k in GRAD_NAMES], ptr(workspace), workspace.numel(), stream)
    return g


# ----------------------------------------------------- Mamba-1 selective scan

def _s6_dims(d) -> S6Dims:
    if isinstance(d, S6Dims):
        return d
    if isinstance(d, dict):
        return S6Dims(**d)
    return S6Dims(*d)


def s6_supported(dstate: int) -> bool:
    return bool(lib.mamba1_s6_supported(dstate))


def s6_workspace_bytes(dims) -> int:
    return int(lib.mamba1_s6_workspace_bytes(ctypes.byref(_s6_dims(dims))))


def s6_check_args(dims, x, delta, A, B, C, h0, y, hT, workspace, ws_bytes) -> int:
    """Host-only validation of a selective-scan call on raw addresses (0 for NULL)."""
    return int(lib.mamba1_s6_check_args(ctypes.byref(_s6_dims(dims)), x, delta, A, B, C, h0, y, hT, workspace,
                                        ws_bytes))


def s6_fwd_ptr(dims, x, delta, A, B, C, h0, y, hT, workspace, ws_bytes, stream: int = 0) -> None:
    """mamba1_s6_fwd on raw device addresses; raises SsdError on a nonzero status."""
    st = lib.mamba1_s6_fwd(ctypes.byref(_s6_dims(dims)), x, delta, A, B, C, h0, y, hT, workspace, ws_bytes, stream)
    if st != 0:
        raise SsdError(st)


def s6_fwd(x, delta, A, B, C, h0=None, *, return_final_state: bool = True, workspace=None):
    """The Mamba-1 selective scan on float32 CUDA tensors: x, delta
    [batch, channels, seqlen], A [channels, dstate], B, C [batch, dstate,
    seqlen], h0 [batch, channels, dstate] or None. Returns ``(y, hT)``."""
    import torch

    for t in (x, delta, A, B, C, h0):
        if t is not None and (t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous()):
            raise ValueError("all tensors must be contiguous float32 GPU tensors")
    bt, D, L = x.shape
    N = A.shape[1]
    if tuple(delta.shape) != (bt, D, L) or tuple(A.shape) != (D, N) or tuple(B.shape) != (bt, N, L) \
            or tuple(C.shape) != (bt, N, L) or (h0 is not None and tuple(h0.shape) != (bt, D, N)):
        raise ValueError("inconsistent shapes")
    dims = S6Dims(bt, L, D, N)
    y = torch.empty_like(x)
    hT = torch.empty((bt, D, N), dtype=torch.float32, device=x.device) if return_final_state else None
    nbytes = s6_workspace_bytes(dims)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    ptr = lambda t: 0 if t is None else t.data_ptr()
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        s6_fwd_ptr(dims, ptr(x), ptr(delta), ptr(A), ptr(B), ptr(C), ptr(h0), ptr(y), ptr(hT), ptr(workspace),
                   workspace.numel(), stream)
    return y, hT


# the selective scan's gradients, in the order mamba1_s6_bwd takes them
S6_GRAD_NAMES = ("dx", "ddelta", "dA", "dB", "dC", "dh0")


def s6_bwd_workspace_bytes(dims) -> int:
    return int(lib.mamba1_s6_bwd_workspace_bytes(ctypes.byref(_s6_dims(dims))))


def s6_bwd_check_args(dims, x, delta, A, B, C, h0, dy, dhT, dx, ddelta, dA, dB, dC, dh0, workspace,
                      ws_bytes) -> int:
    """Host-only validation of a selective-scan backward call on raw addresses (0 for NULL)."""
    return int(lib.mamba1_s6_bwd_check_args(ctypes.byref(_s6_dims(dims)), x, delta, A, B, C, h0, dy, dhT, dx,
                                            ddelta, dA, dB, dC, dh0, workspace, ws_bytes))


def s6_bwd_ptr(dims, x, delta, A, B, C, h0, dy, dhT, dx, ddelta, dA, dB, dC, dh0, workspace, ws_bytes,
               stream: int = 0) -> None:
    """mamba1_s6_bwd on raw device addresses; raises SsdError on a nonzero status."""
    st = lib.mamba1_s6_bwd(ctypes.byref(_s6_dims(dims)), x, delta, A, B, C, h0, dy, dhT, dx, ddelta, dA, dB, dC,
                           dh0, workspace, ws_bytes, stream)
    if st != 0:
        raise SsdError(st)


def s6_bwd(x, delta, A, B, C, dy, h0=None, dhT=None, *, workspace=None):
    """Gradients of the selective scan on float32 CUDA tensors (shapes as
    ``s6_fwd``; dy like x, dhT like h0 or None). Returns a dict with dx,
    ddelta, dA, dB, dC and dh0."""
    import torch

    for t in (x, delta, A, B, C, dy, h0, dhT):
        if t is not None and (t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous()):
            raise ValueError("all tensors must be contiguous float32 GPU tensors")
    bt, D, L = x.shape
    N = A.shape[1]
    for t, shape in ((delta, (bt, D, L)), (A, (D, N)), (B, (bt, N, L)), (C, (bt, N, L)), (dy, (bt, D, L)),
                     (h0, (bt, D, N)), (dhT, (bt, D, N))):
        if t is not None and tuple(t.shape) != shape:
            raise ValueError("inconsistent shapes")
    dims = S6Dims(bt, L, D, N)
    g = {"dx": torch.empty_like(x), "ddelta": torch.empty_like(x), "dA": torch.empty_like(A),
         "dB": torch.empty_like(B), "dC": torch.empty_like(B),
         "dh0": torch.empty((bt, D, N), dtype=torch.float32, device=x.device)}
    nbytes = s6_bwd_workspace_bytes(dims)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    ptr = lambda t: 0 if t is None else t.data_ptr()
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        s6_bwd_ptr(dims, ptr(x), ptr(delta), ptr(A), ptr(B), ptr(C), ptr(h0), ptr(dy), ptr(dhT),
                   *[ptr(g[k]) for k in S6_GRAD_NAMES], ptr(workspace), workspace.numel(), stream)
    return g
