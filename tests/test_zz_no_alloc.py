"""qgemv_batch_scratch, the entry point that allocates nothing (its workspace is the
library's static device scratch), against qgemv_batch with a caller-allocated workspace:
called through the C ABI on shapes whose kernels use the workspace (staged activation tiles
and column-split partial sums on the float matrix cores; column-split partial sums on the
integer matrix cores), several calls in a row with later ones smaller, so that each call runs
on what the previous one left in the scratch. Each y must be bit-identical to qgemv_batch's
(the same kernels in the same order) and within the oracle's bound
|y - y_ref| <= 1e-5 sum |w||x|."""

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")

# (rows, cols, vectors): route, and what the workspace holds
CALLS = [
    (3000, 2048, 40),     # float matrix cores: tiles + 8 column splits of partial sums (4.1 MB)
    (700, 4096, 12),      # integer matrix cores: 2 column splits of partial sums (67 KB)
    (200, 1024, 20),      # float matrix cores again, smaller than the first (1.1 MB)
]


def _say(*a):
    print("[no-alloc]", *a, flush=True)


def test_scratch_entry_point_equals_batch_with_workspace():
    import torch
    import block_quantized_weight_act_amd as qg
    gu.require_gpu()
    for rows, cols, nvec in CALLS:
        _say("call", rows, cols, nvec, qg.qgemv_route("q4k", rows, cols, nvec))
        need = qg.qgemv_workspace_bytes("q4k", rows, cols, nvec)
        assert 0 < need <= qg.SCRATCH_BYTES
        rng = np.random.default_rng(rows + cols + nvec)
        wbuf = oracle.quantize("q4k", (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32))
        x = rng.standard_normal((nvec, cols)).astype(np.float32)
        rq, rd = oracle.quantize_act(x)
        ref = oracle.gemv("q4k", wbuf, rows, cols, rq, rd)
        w = gu.dev(wbuf)
        xq, xd = gu.dev(rq), gu.dev(rd)
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=gu.DEV)
        y_ws = torch.full((nvec, rows), float("nan"), dtype=torch.float32, device=gu.DEV)
        qg.qgemv_batch("q4k", w, xq, xd, y_ws, rows, cols, nvec, workspace=ws)
        y_sc = torch.full_like(y_ws, float("nan"))
        qg.qgemv_batch_scratch("q4k", w, xq, xd, y_sc, rows, cols, nvec)
        a, b = gu.host(y_ws), gu.host(y_sc)
        gu.assert_within_bound(b, ref)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_scratch_entry_point_refuses_shapes_beyond_the_scratch():
    import torch
    import block_quantized_weight_act_amd as qg
    gu.require_gpu()
    rows, cols, nvec = 128, 65536, 256
    assert qg.qgemv_workspace_bytes("q4k", rows, cols, nvec) > qg.SCRATCH_BYTES
    w = torch.zeros(qg.qgemv_weight_bytes("q4k", rows, cols), dtype=torch.uint8, device=gu.DEV)
    xq = torch.zeros((nvec, cols), dtype=torch.int8, device=gu.DEV)
    xd = torch.zeros((nvec, cols // 32), dtype=torch.float32, device=gu.DEV)
    y = torch.full((nvec, rows), 7.0, dtype=torch.float32, device=gu.DEV)
    with pytest.raises(qg.QgemvError) as e:
        qg.qgemv_batch_scratch("q4k", w, xq, xd, y, rows, cols, nvec)
    assert e.value.status == 3
    assert bool((y == 7.0).all())                # nothing ran
