"""The Q6_K 2048 x 8192 batch-1 workload (a short, wide matrix) with its columns split into
chunks of whole 32-column blocks (genie-ai-runtime, "v1.3.0": split the reduction dimension
when rows alone under-fill the GPU, then add the partial results in a separate pass).

The library's own plan for this shape covers each 8192-column row in one pass (measured
faster), so the split forms are forced through explicit plans, at the full shape:
  - with S <= a workgroup's waves: the split inside the workgroup (one launch, the chunks' row
    sums added in LDS in ascending chunk order), from codes and fused (the workgroup quantizing
    every chunk of the row into LDS first);
  - with more chunks: partial sums in the workspace and the ordered reduce launch (the
    atomic-free two-pass form), from codes and fused (each workgroup quantizing its chunk).
Every y lies within the oracle's bound |y - y_ref| <= 1e-5 sum |w||x|; the fused y is
bit-identical to the from-codes y of the same plan (the same chunks, added in the same order);
the fused codes, and the integer partials P and S, are the oracle's bit for bit."""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")

WL = synth.WORKLOADS["q6k_2048x8192"]

# (lanes per row, chunks per lane, waves per workgroup, workgroups per column chunk)
IN_WORKGROUP = [(64, 2, 4, 256), (64, 2, 8, 128), (64, 1, 4, 128), (32, 2, 4, 128),
                (32, 4, 8, 128)]                                    # S = 2, 2, 4, 4, 2
TWO_PASS = [(32, 1, 4, 64), (16, 2, 4, 64), (16, 1, 4, 64), (8, 4, 4, 32)]   # S = 8, 8, 16, 8


def _say(*a):
    print("[c2-split]", *a, flush=True)


@pytest.fixture(scope="module")
def c2():
    gu.require_gpu()
    _say("oracle reference", WL.rows, WL.cols)
    wbuf = oracle.quantize("q6k", WL.weight_block(0, WL.rows))
    x = WL.activations()
    rq, rd = oracle.quantize_act(x)
    ref = oracle.gemv("q6k", wbuf, WL.rows, WL.cols, rq, rd, partials=True)
    xq, xd = gu.quantize_act(x)
    assert np.array_equal(gu.host(xq), rq)
    return dict(wbuf=wbuf, wd=gu.dev(wbuf), xt=gu.dev(x), xq=xq, xd=xd, rq=rq, rd=rd, ref=ref)


def _plan(t, nc, wv, b):
    return dict(lanes_per_row=t, chunks_per_lane=nc, waves_per_block=wv, blocks=b)


def _splits(p):
    return -(-(WL.cols // 32) // (p["lanes_per_row"] * p["chunks_per_lane"]))


def _both_forms(c2, plan):
    """y from codes (qgemv_batch_plan) and y of the fused form (qgemv_fused_plan),
    each through a workspace filled with 0xFF (NaN) first; and the fused form's codes."""
    import torch
    import block_quantized_weight_act_amd as qg
    rows, cols = WL.rows, WL.cols
    nbytes = qg.qgemv_plan_workspace_bytes(plan, rows, cols, 1)
    assert nbytes == _splits(plan) * rows * 4
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=gu.DEV)
    y_codes = torch.full((1, rows), float("nan"), dtype=torch.float32, device=gu.DEV)
    qg.qgemv_batch_plan("q6k", c2["wd"], c2["xq"], c2["xd"], y_codes, rows, cols, 1, plan,
                        workspace=ws)
    ws.fill_(0xFF)
    y_fused = torch.full_like(y_codes, float("nan"))
    xq_out = torch.zeros((1, cols), dtype=torch.int8, device=gu.DEV)
    xd_out = torch.zeros((1, cols // 32), dtype=torch.float32, device=gu.DEV)
    qg.qgemv_fused_plan("q6k", c2["wd"], c2["xt"], y_fused, rows, cols, 1, plan, xq_out=xq_out,
                        xd_out=xd_out, workspace=ws)
    assert np.array_equal(gu.host(xq_out), c2["rq"])
    assert np.array_equal(gu.host(xd_out).view(np.uint32), c2["rd"].view(np.uint32))
    return gu.host(y_codes), gu.host(y_fused)


def test_c2_partials_bit_exact_and_default_plan(c2):
    import block_quantized_weight_act_amd as qg
    plan = qg.qgemv_plan_for("q6k", WL.rows, WL.cols, 1)
    _say("default plan", plan)
    assert plan["splits"] == 1 and plan["lanes_per_row"] * plan["chunks_per_lane"] == 256
    P, S = gu.partials("q6k", c2["wd"], c2["xq"], c2["xd"], WL.rows, WL.cols, 1)
    assert np.array_equal(P, c2["ref"]["P"])
    assert np.array_equal(S, oracle.block_sums(c2["rq"]))
    gu.assert_within_bound(gu.gemv("q6k", c2["wd"], c2["xq"], c2["xd"], WL.rows, WL.cols, 1),
                           c2["ref"])


@pytest.mark.parametrize("t,nc,wv,b", IN_WORKGROUP)
def test_c2_split_inside_workgroup_equals_two_pass(c2, t, nc, wv, b):
    plan = _plan(t, nc, wv, b)
    _say("in-workgroup", plan, "S =", _splits(plan))
    assert 2 <= _splits(plan) <= wv
    y_codes, y_fused = _both_forms(c2, plan)
    gu.assert_within_bound(y_codes, c2["ref"])
    assert np.array_equal(y_fused.view(np.uint32), y_codes.view(np.uint32))


@pytest.mark.parametrize("t,nc,wv,b", TWO_PASS)
def test_c2_split_two_pass(c2, t, nc, wv, b):
    plan = _plan(t, nc, wv, b)
    _say("two-pass", plan, "S =", _splits(plan))
    assert _splits(plan) > wv
    y_codes, y_fused = _both_forms(c2, plan)
    gu.assert_within_bound(y_codes, c2["ref"])
    assert np.array_equal(y_fused.view(np.uint32), y_codes.view(np.uint32))
