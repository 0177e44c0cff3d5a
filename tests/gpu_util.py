"""Helpers for the GPU parity tests: move numpy arrays to the device and call the HIP
library through its C-ABI binding. Nothing here computes the method."""

from __future__ import annotations

import numpy as np
import torch

import block_quantized_weight_act_amd as qg

DEV = "cuda:0"


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU (torch.cuda.is_available() is False)")


def dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def quantize_act(x: np.ndarray):
    x = np.ascontiguousarray(np.atleast_2d(x), np.float32)
    nvec, cols = x.shape
    xt = dev(x)
    xq = torch.empty((nvec, cols), dtype=torch.int8, device=DEV)
    xd = torch.empty((nvec, cols // 32), dtype=torch.float32, device=DEV)
    qg.qgemv_quantize_act(xt, xq, xd, cols, nvec)
    return xq, xd


def quantize_weights(wtype: str, w: np.ndarray) -> torch.Tensor:
    rows, cols = w.shape
    out = torch.empty(qg.qgemv_weight_bytes(wtype, rows, cols), dtype=torch.uint8, device=DEV)
    qg.qgemv_quantize_weights(wtype, dev(np.asarray(w, np.float32)), out, rows, cols)
    return out


def gemv(wtype: str, w, xq, xd, rows: int, cols: int, nvec: int, plan=None) -> np.ndarray:
    wt = w if isinstance(w, torch.Tensor) else dev(w)
    xq = xq if isinstance(xq, torch.Tensor) else dev(xq)
    xd = xd if isinstance(xd, torch.Tensor) else dev(xd)
    y = torch.full((nvec, rows), float("nan"), dtype=torch.float32, device=DEV)
    if plan is None:
        nbytes = qg.qgemv_workspace_bytes(wtype, rows, cols, nvec)
    else:
        nbytes = qg.qgemv_plan_workspace_bytes(plan, rows, cols, nvec)
    ws = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=DEV) if nbytes else None
    if plan is not None:
        qg.qgemv_batch_plan(wtype, wt, xq, xd, y, rows, cols, nvec, plan, workspace=ws)
    elif nvec == 1 and wtype == "q4k":
        qg.qgemv_q4k(wt, xq, xd, y, rows, cols, workspace=ws)
    elif nvec == 1 and wtype == "q6k":
        qg.qgemv_q6k(wt, xq, xd, y, rows, cols, workspace=ws)
    else:
        qg.qgemv_batch(wtype, wt, xq, xd, y, rows, cols, nvec, workspace=ws)
    return host(y)


def partials(wtype: str, w, xq, xd, rows: int, cols: int, nvec: int):
    wt = w if isinstance(w, torch.Tensor) else dev(w)
    xq = xq if isinstance(xq, torch.Tensor) else dev(xq)
    xd = xd if isinstance(xd, torch.Tensor) else dev(xd)
    nsub = cols // 16 if wtype == "q6k" else cols // 32
    P = torch.full((nvec, rows, nsub), -(2 ** 31), dtype=torch.int32, device=DEV)
    S = torch.full((nvec, cols // 32), -(2 ** 31), dtype=torch.int32, device=DEV)
    nbytes = qg.qgemv_workspace_bytes(wtype, rows, cols, nvec)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV) if nbytes else None
    qg.qgemv_debug_partials(wtype, wt, xq, xd, P, S, rows, cols, nvec, workspace=ws)
    return host(P), host(S)


def assert_within_bound(y_gpu: np.ndarray, ref: dict, rel: float = 1e-5):
    """|y - y_ref| <= rel * sum_i |w_i| |x_i| for every output."""
    y_ref, bound = ref["y"], ref["bound"]
    assert y_gpu.shape == y_ref.shape
    assert np.all(np.isfinite(y_gpu))
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bad = err > rel * bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("y outside the bound at %s: gpu %r ref %r bound %r (%d bad)" % (
            tuple(i), float(y_gpu[tuple(i)]), float(y_ref[tuple(i)]), float(bound[tuple(i)]),
            int(bad.sum())))
