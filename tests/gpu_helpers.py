"""Shared helpers for the GPU tests: device transfer, calls through the C ABI,
workspace views and the parity tolerances.

Tolerances (stated with the build's targets):
  fp32 io: max|y - y_ref| / max|y_ref| <= 1e-5 (normwise, per tensor)
  bf16 io: |y - y_ref| <= 1e-2 + 2e-2 * |y_ref| for every element
The reference is the fp64 oracle on the same (already bf16-rounded) inputs.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import state_space_sequence_ssd_amd as ssd
from state_space_sequence_ssd_amd import BF16, F32, Dims

F32_TOL = 1e-5
BF16_ATOL, BF16_RTOL = 1e-2, 2e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp: dict, io: str, dev="cuda:0") -> dict:
    """numpy inputs from workloads.generate -> contiguous torch CUDA tensors."""
    out = {}
    for k in ("x", "B", "C"):
        if io == "bf16":
            bits = inp[k + "_bits"] if k + "_bits" in inp else None
            if bits is None:
                from workloads import round_to_bf16
                bits = round_to_bf16(inp[k])[1]
            out[k] = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(inp[k], dtype=np.float32)).to(dev)
    for k in ("dt", "A", "D"):
        out[k] = torch.from_numpy(np.ascontiguousarray(inp[k], dtype=np.float32)).to(dev)
    init = inp.get("init_state")
    out["init_state"] = None if init is None else torch.from_numpy(np.ascontiguousarray(init, dtype=np.float32)).to(dev)
    return out


def run(dev_inp: dict, chunk: int, keep_workspace=False, init_state="default", final=True, path=0):
    """Call the library (``path``: a PATH_* kernel sequence, 0 = the library's
    choice); optionally return the workspace for per-kernel checks."""
    init = dev_inp["init_state"] if init_state == "default" else init_state
    x = dev_inp["x"]
    io = BF16 if x.dtype == torch.bfloat16 else F32
    bt, T, H, P = x.shape
    G, N = dev_inp["B"].shape[2:]
    dims = Dims(bt, T, H, P, N, G, chunk)
    L = ssd.workspace_layout(dims, io | path)
    ws = torch.empty(max(L.total_bytes, 1), dtype=torch.uint8, device=x.device)
    y, fin = ssd.ssd_fwd(x, dev_inp["dt"], dev_inp["A"], dev_inp["B"], dev_inp["C"], dev_inp["D"], chunk,
                         init, return_final_state=final, workspace=ws, path=path)
    torch.cuda.synchronize()
    if keep_workspace:
        return y, fin, ws, L, dims
    return y, fin


def workspace_views(ws, L, dims, io):
    """The intermediates, laid out as documented in include/mamba2_ssd.h."""
    bt, H, P, N, nc = dims.batch, dims.nheads, dims.headdim, dims.dstate, L.nchunks
    Tp = nc * dims.chunk

    def view(off, count, dtype):
        nbytes = count * torch.tensor([], dtype=dtype).element_size()
        return ws[off:off + nbytes].view(dtype)

    if io == BF16:
        # (hi, lo) bf16 pairs: per row, per aligned group of 8 columns, 8 hi then 8 lo
        pairs = view(L.hprev_offset, bt * H * nc * P * N * 2, torch.bfloat16).float()
        pairs = pairs.view(bt, H, nc, P, N // 8, 2, 8)
        hprev = (pairs[..., 0, :] + pairs[..., 1, :]).reshape(bt, H, nc, P, N)
    else:
        hprev = view(L.hprev_offset, bt * H * nc * P * N, torch.float32).view(bt, H, nc, P, N)
    return {
        "gcum": view(L.gcum_offset, bt * H * Tp, torch.float32).view(bt, H, Tp),
        "dtt": view(L.dtt_offset, bt * H * Tp, torch.float32).view(bt, H, Tp),
        "wst": view(L.wst_offset, bt * H * Tp, torch.float32).view(bt, H, Tp),
        "states": view(L.states_offset, bt * H * nc * P * N, torch.float32).view(bt, H, nc, P, N),
        "hprev": hprev,
    }


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_close(got, ref, io: str, what: str):
    """Assert the stated tolerance; returns a short error summary string."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    if io == "f32":
        den = max(float(np.max(np.abs(ref))), 1e-30)
        rel = float(np.max(err)) / den
        assert rel <= F32_TOL, f"{what}: normwise relative error {rel:.3e} > {F32_TOL}"
        return f"{what}: normwise rel err {rel:.2e}"
    bound = BF16_ATOL + BF16_RTOL * np.abs(ref)
    ratio = err / bound
    worst = float(np.max(ratio)) if ratio.size else 0.0
    nbad = int(np.sum(ratio > 1.0))
    if nbad:
        i = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(f"{what}: {nbad} of {ratio.size} elements outside 1e-2 + 2e-2|ref| "
                             f"(worst at {i}: got {got[i]:.6g}, ref {ref[i]:.6g})")
    normwise = float(np.max(err)) / max(float(np.max(np.abs(ref))), 1e-30)
    return f"{what}: worst |err|/bound {worst:.3f}, normwise {normwise:.2e}"
