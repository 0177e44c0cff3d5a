"""Host-side planning against the documented rules, on random shapes (no GPU, no launches):
the per-shape plan's invariants and its workspace, the route qgemv_batch takes (vector kernels,
integer or float matrix cores, groups of 8), and the multi-matrix lane geometry. The rules are
restated here from their documentation in include/qgemv.h, so a change of the library's rule that
the documentation does not follow fails here."""

import math

import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import block_quantized_weight_act_amd as qg  # noqa: E402

pytestmark = pytest.mark.skipif(not __import__("os").path.exists(qg.library_path),
                                reason="library not built")

WTYPES = ["q4k", "q6k", "q40", "q80"]
BLOCK_COLS = {"q4k": 256, "q6k": 256, "q40": 32, "q80": 32}
BYTES_PER_BLOCK = {"q4k": 144, "q6k": 210, "q40": 18, "q80": 36}
MI = 1 << 20
# tensors from which qgemv_batch takes the integer matrix cores for Q4_K with 3..8 vectors
I8_MIN_MIB = {3: 128, 4: 96, 5: 48, 6: 32, 7: 24, 8: 16}


@st.composite
def shapes(draw, max_vec=8):
    wtype = draw(st.sampled_from(WTYPES))
    blocks = draw(st.integers(1, 64 if BLOCK_COLS[wtype] == 256 else 512))
    cols = blocks * BLOCK_COLS[wtype]
    rows = draw(st.one_of(st.integers(1, 5000), st.integers(5000, 400000)))
    nvec = draw(st.integers(1, max_vec))
    return wtype, rows, cols, nvec


def weight_bytes(wtype, rows, cols):
    return rows * cols // BLOCK_COLS[wtype] * BYTES_PER_BLOCK[wtype]


@settings(max_examples=300, deadline=None)
@given(shapes())
def test_plan_invariants_and_workspace(shape):
    wtype, rows, cols, nvec = shape
    assert qg.qgemv_weight_bytes(wtype, rows, cols) == weight_bytes(wtype, rows, cols)
    p = qg.qgemv_plan_for(wtype, rows, cols, nvec)
    t, nc, w, b, s = (p["lanes_per_row"], p["chunks_per_lane"], p["waves_per_block"], p["blocks"],
                      p["splits"])
    assert t in (8, 16, 32, 64) and 1 <= nc <= 4 and nvec * nc <= 8
    assert s == math.ceil(cols // 32 / (t * nc))
    assert w in (4, 8) and (w == 4 or nvec * t * nc >= 128)
    assert b >= 1
    # the vector kernels' workspace: the partial sums of the column chunks, none unsplit
    expect = s * nvec * rows * 4 if s > 1 else 0
    assert qg.qgemv_plan_workspace_bytes(p, rows, cols, nvec) == expect
    if qg.qgemv_route(wtype, rows, cols, nvec) == "vector":
        assert qg.qgemv_workspace_bytes(wtype, rows, cols, nvec) == expect
    # without code outputs the fused form is always one launch
    assert qg.qgemv_fused_launches(wtype, rows, cols, nvec, False) == 1


def few_kernel_rule(wtype, rows, cols, nvec):
    """Where qgemv_batch takes the few-vector integer matrix-core kernel (QGEMV_ROUTE_MC32 with
    up to 16 vectors), as include/qgemv.h documents it: rows of up to 2048 columns (one split)
    unless noted; with 1..8 vectors Q4_0 from 4 vectors on >= 32 Mi weights (3 from 256 Mi; 8
    on wider rows), Q6_K from 4 vectors on 256 Mi weights and with 8 from 64 Mi, Q8_0 with 8
    from 256 Mi, Q4_K with 4 on tensors of 16 to 96 MiB; with 9..16 vectors (any width) from
    16 Mi weights, Q8_0 with 9..15 vectors not on 48 to 256 Mi, Q4_K only with 9..12 vectors
    below 128 MiB."""
    weights = rows * cols
    wb = weight_bytes(wtype, rows, cols)
    one = cols <= 2048
    if nvec <= 8:
        if wtype == "q40":
            return weights >= 32 * MI and nvec >= (8 if not one else (3 if weights >= 256 * MI else 4))
        if wtype == "q6k":
            return one and ((weights >= 256 * MI and nvec >= 4) or (weights >= 64 * MI and nvec >= 8))
        if wtype == "q80":
            return one and weights >= 256 * MI and nvec >= 8
        return one and nvec == 4 and 16 * MI <= wb < 96 * MI
    if nvec > 16 or weights < 16 * MI:
        return False
    if wtype == "q80":
        return nvec >= 16 or weights < 48 * MI or weights >= 256 * MI
    if wtype == "q4k":
        return nvec <= 12 and wb < 128 * MI
    return True


@settings(max_examples=400, deadline=None)
@given(shapes(max_vec=256))
def test_route_follows_the_documented_rule(shape):
    wtype, rows, cols, nvec = shape
    route = qg.qgemv_route(wtype, rows, cols, nvec)
    wb = weight_bytes(wtype, rows, cols)
    weights = rows * cols
    few = few_kernel_rule(wtype, rows, cols, nvec)
    if wtype == "q4k":
        if nvec <= 8:
            i8 = nvec >= 3 and wb >= I8_MIN_MIB[nvec] * MI
            expect = "i8mc" if i8 else ("mc32" if few else "vector")
        elif nvec <= 16:
            expect = "mc32" if few else "i8mc"
        else:
            expect = "mc"
    elif nvec <= 8:
        expect = "mc32" if few else "vector"
    else:
        mc = few or nvec >= 32 or (nvec >= 16 and weights >= 24 * MI) or weights >= 48 * MI
        expect = "mc32" if mc else "grouped"
    assert route == expect, (wtype, rows, cols, nvec, route)


def multi_rule(cols, nvec):
    """Lanes per row and chunks per lane of a multi-matrix launch: the fewest idle lanes among
    the geometries covering a row in one pass (more chunks per lane preferred, at most 3 with 2
    vectors); else the one-matrix rule (each further pass priced as 2% of the lanes idle, 15%
    from 5 vectors) among the geometries with at most a workgroup's waves of passes (8 when
    nvec * lanes * chunks >= 128, else 4)."""
    nchunks = cols // 32
    split_cost = 0.15 if nvec >= 5 else 0.02
    for one_pass in (True, False):
        best, best_cost = None, 1e30
        for nc in range(1, 5):
            if nvec * nc > 8 or (nvec == 2 and nc > 3):
                break
            for t in (8, 16, 32, 64):
                passes = -(-nchunks // (t * nc))
                if one_pass and passes > 1:
                    continue
                if passes > (8 if nvec * t * nc >= 128 else 4):
                    continue
                cost = 1.0 - nchunks / (passes * t * nc) + split_cost * (passes - 1) - 0.01 * nc
                if cost < best_cost - 1e-12:
                    best, best_cost = (t, nc), cost
        if best is not None:
            return best
    return None


@settings(max_examples=300, deadline=None)
@given(st.integers(1, 2500), st.integers(1, 8))
def test_multi_geometry_follows_the_documented_rule(blocks, nvec):
    cols = 32 * blocks
    expect = multi_rule(cols, nvec)
    if expect is None:
        with pytest.raises(qg.QgemvError):
            qg.qgemv_multi_geometry(cols, nvec)
    else:
        assert qg.qgemv_multi_geometry(cols, nvec) == expect
