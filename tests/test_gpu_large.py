"""GPU parity on tensors larger than 4 GiB, so that every plane offset, row offset and workspace
offset of the kernels needs 64 bits: Q4_K, Q6_K, Q4_0 and Q8_0 with 327680 rows of 32768
columns (6.0 to 11.4 GB; Q4_K's header plane starts at 5.4 GB), through the one-vector kernel,
the fused one-launch kernel, the integer matrix-core kernels (8 and 16 vectors) and the float
matrix-core kernel (64 vectors).

The tensor is U = 64 rows quantized by the oracle and repeated (plane by plane, on the GPU), so
row r equals row r % U and the oracle's y for the U rows, repeated, is the reference for every
row; the integer partials are checked on rows sampled across the whole tensor."""

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")

ROWS, COLS, U = 327680, 32768, 64
WIDTHS = {"q4k": [128, 16], "q6k": [128, 64, 16, 2], "q40": [16, 2], "q80": [16, 16, 4]}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.require_gpu()


def _say(*a):
    print("[large]", *a, flush=True)


def _big_tensor(wtype, small):
    """The ROWS-row tensor whose row r is row r % U of the U-row tensor `small`, built on the
    GPU plane by plane."""
    import torch
    import block_quantized_weight_act_amd as qg
    nb = COLS // (32 if wtype in ("q40", "q80") else 256)
    big = torch.empty(qg.qgemv_weight_bytes(wtype, ROWS, COLS), dtype=torch.uint8, device=gu.DEV)
    assert big.numel() > (1 << 32)
    sm = gu.dev(small)
    off_b = off_s = 0
    for wd in WIDTHS[wtype]:
        per_row = nb * wd
        src = sm[off_s:off_s + U * per_row].view(1, U * per_row)
        dst = big[off_b:off_b + ROWS * per_row].view(ROWS // U, U * per_row)
        dst.copy_(src.expand(ROWS // U, U * per_row))
        off_s += U * per_row
        off_b += ROWS * per_row
    assert off_b == big.numel()
    return big


CASES = [("q4k", 1), ("q4k", 8), ("q4k", 16), ("q4k", 64), ("q6k", 1), ("q6k", 8), ("q6k", 16),
         ("q40", 1), ("q40", 8), ("q40", 16), ("q80", 1), ("q80", 8), ("q80", 16)]


@pytest.mark.parametrize("wtype", ["q4k", "q6k", "q40", "q80"])
def test_beyond_4gib(wtype):
    import torch
    import block_quantized_weight_act_amd as qg
    rng = np.random.default_rng({"q4k": 1, "q6k": 2, "q40": 3, "q80": 4}[wtype])
    w = (rng.standard_normal((U, COLS)) * 0.02).astype(np.float32)
    small = oracle.quantize(wtype, w)
    big = _big_tensor(wtype, small)
    for wt, nvec in CASES:
        if wt != wtype:
            continue
        _say(wtype, ROWS, COLS, nvec, qg.qgemv_route(wtype, ROWS, COLS, nvec))
        x = (rng.standard_normal((nvec, COLS)) * rng.choice([0.01, 1.0, 30.0], size=(nvec, 1))
             ).astype(np.float32)
        rq, rd = oracle.quantize_act(x)
        ref_u = oracle.gemv(wtype, small, U, COLS, rq, rd)
        ref = {k: np.tile(ref_u[k], (1, ROWS // U)) for k in ("y", "bound")}
        xq, xd = gu.quantize_act(x)
        gu.assert_within_bound(gu.gemv(wtype, big, xq, xd, ROWS, COLS, nvec), ref)
        if nvec == 8 and wtype != "q4k":
            # the few-vector matrix-core kernel itself, whatever the route
            y = torch.full((nvec, ROWS), float("nan"), dtype=torch.float32, device=gu.DEV)
            nbytes = qg.qgemv_mc32_workspace_bytes(wtype, ROWS, COLS, nvec)
            ws = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=gu.DEV) if nbytes else None
            qg.qgemv_batch_mc32(wtype, big, xq, xd, y, ROWS, COLS, nvec, workspace=ws)
            gu.assert_within_bound(gu.host(y), ref)
            del y, ws
        if nvec == 1:
            # the fused one-launch kernel (no code outputs)
            y = torch.full((1, ROWS), float("nan"), dtype=torch.float32, device=gu.DEV)
            nbytes = qg.qgemv_workspace_bytes(wtype, ROWS, COLS, 1)
            ws = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=gu.DEV) if nbytes else None
            qg.qgemv_fused(wtype, big, gu.dev(x), y, ROWS, COLS, 1, workspace=ws)
            gu.assert_within_bound(gu.host(y), ref)
        if nvec in (1, 8, 16):
            # integer partials on rows sampled over the whole tensor (the last rows included),
            # gathered on the GPU (the whole array is up to 43 GB); with 8 vectors those of the
            # few-vector matrix-core kernel whatever the route
            nsub = COLS // 16 if wtype == "q6k" else COLS // 32
            P = torch.full((nvec, ROWS, nsub), -(2 ** 31), dtype=torch.int32, device=gu.DEV)
            S = torch.empty((nvec, COLS // 32), dtype=torch.int32, device=gu.DEV)
            nbytes = qg.qgemv_workspace_bytes(wtype, ROWS, COLS, nvec)
            ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=gu.DEV) if nbytes else None
            if nvec == 8 and wtype != "q4k":
                qg.qgemv_debug_partials_mc32(wtype, big, xq, xd, P, S, ROWS, COLS, nvec)
            else:
                qg.qgemv_debug_partials(wtype, big, xq, xd, P, S, ROWS, COLS, nvec, workspace=ws)
            rows = np.concatenate([np.arange(0, ROWS, 4099), np.arange(ROWS - U, ROWS)])
            got = gu.host(P[:, torch.from_numpy(rows).to(gu.DEV)])
            del P, S, ws
            ref = oracle.gemv(wtype, small, U, COLS, rq, rd, partials=True)
            assert np.array_equal(got, ref["P"][:, rows % U])
        del xq, xd
    del big
    torch.cuda.empty_cache()
