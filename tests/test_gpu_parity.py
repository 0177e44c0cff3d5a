"""GPU parity: the HIP library (called through its C ABI) against the CPU oracle.

Bars: activation codes and scales, weight bytes and the integer partials P and S are
bit-exact; y satisfies |y - y_ref| <= 1e-5 * sum_i |w_i| |x_i| per output (w the
dequantized weights, x the dequantized activations), with y_ref and the bound computed by
the oracle in float64.
"""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.require_gpu()


def _say(*a):
    print("[parity]", *a, flush=True)


def _quant(wtype, w, negate=False):
    """The oracle's tensor of w in any format (Q6_K optionally with negated sub-scales)."""
    if wtype == "q6k":
        return oracle.quantize_q6k(w, negate_scales=negate)
    return oracle.quantize(wtype, w)


ALL = ["q4k", "q6k", "q40", "q80"]


# --------------------------------------------------------------- activations --
@pytest.mark.parametrize("nvec,cols", [(1, 32), (1, 96), (2, 1536), (8, 2048), (3, 8192),
                                       (1, 32 * 1001)])
def test_quantize_act_bitexact(nvec, cols):
    _say("quantize_act", nvec, cols)
    rng = np.random.default_rng(cols + nvec)
    x = rng.standard_normal((nvec, cols)).astype(np.float32)
    x[0, :32] = 0.0                                    # all-zero block
    if cols >= 96:
        x[0, 32:64] *= np.float32(1e-30)               # tiny block
        x[0, 64:96] = np.float32(7.0)                  # constant block
    if nvec > 1:
        x[1] *= np.float32(1e4)
    xq, xd = gu.quantize_act(x)
    rq, rd = oracle.quantize_act(x)
    assert np.array_equal(gu.host(xq), rq)
    assert np.array_equal(gu.host(xd).view(np.uint32), rd.view(np.uint32))


def test_quantize_act_hand_worked_ties():
    import oracle_pins
    cases = oracle_pins.read_act_cases()
    x = np.stack([c[0] for c in cases]).reshape(1, -1)
    xq, xd = gu.quantize_act(x)
    assert np.array_equal(gu.host(xq).reshape(len(cases), 32), np.stack([c[1] for c in cases]))
    assert np.array_equal(gu.host(xd)[0], np.array([c[2] for c in cases], np.float32))


def _tiny_blocks(nvec, cols, seed):
    """Activations with blocks whose maximum lies below, at and above 127 / FLT_MAX (about
    3.73e-37), where 127 / amax stops being a finite float32, each with a zero element."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((nvec, cols)).astype(np.float32)
    for b, amax in enumerate([1e-37, 3.7e-37, 3.8e-37, 2e-38, 1.5e-45, 1e-30]):
        blk = (rng.uniform(-1.0, 1.0, 32) * amax).astype(np.float32)
        blk[5] = np.float32(-amax)
        blk[9] = 0.0
        x[b % nvec, 32 * (2 * b + 1):32 * (2 * b + 2)] = blk
    return x


def test_quantize_act_overflowing_inverse():
    """Blocks whose 127 / amax overflows float32 get the codes 0 (the amax = 0 rule) on every
    GPU quantizer: qgemv_quantize_act, the fused one-launch kernels of all four formats, the
    integer matrix-core kernel's own quantization, and the Q8_0 weight quantizer; codes and
    scales bit for bit the oracle's, y within its bound."""
    import torch
    import block_quantized_weight_act_amd as qg
    nvec, cols = 2, 2048
    x = _tiny_blocks(nvec, cols, 3)
    rq, rd = oracle.quantize_act(x)
    assert not rq[0, 32:64].any() and not rq[1, 96:128].any()       # 1e-37 and 3.7e-37 blocks
    xq, xd = gu.quantize_act(x)
    assert np.array_equal(gu.host(xq), rq)
    assert np.array_equal(gu.host(xd).view(np.uint32), rd.view(np.uint32))
    xt = gu.dev(x)
    rng = np.random.default_rng(4)
    rows = 300
    for wtype in ALL:
        _say("overflowing inverse, fused", wtype)
        wbuf = _quant(wtype, (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32))
        ref = oracle.gemv(wtype, wbuf, rows, cols, rq, rd)
        w = gu.dev(wbuf)
        assert qg.qgemv_fused_launches(wtype, rows, cols, nvec) == 1
        y = torch.full((nvec, rows), float("nan"), dtype=torch.float32, device=gu.DEV)
        xq_out = torch.zeros((nvec, cols), dtype=torch.int8, device=gu.DEV)
        xd_out = torch.zeros((nvec, cols // 32), dtype=torch.float32, device=gu.DEV)
        qg.qgemv_fused(wtype, w, xt, y, rows, cols, nvec, xq_out=xq_out, xd_out=xd_out)
        gu.assert_within_bound(gu.host(y), ref)
        assert np.array_equal(gu.host(xq_out), rq)
        assert np.array_equal(gu.host(xd_out).view(np.uint32), rd.view(np.uint32))
        if wtype == "q4k":
            y.fill_(float("nan"))
            xq_out.zero_()
            xd_out.zero_()
            qg.qgemv_fused_i8mc(w, xt, y, rows, cols, nvec, xq_out=xq_out, xd_out=xd_out)
            gu.assert_within_bound(gu.host(y), ref)
            assert np.array_equal(gu.host(xq_out), rq)
            assert np.array_equal(gu.host(xd_out).view(np.uint32), rd.view(np.uint32))
    # the Q8_0 weight quantizer applies the same rule to each block of 32 weights
    wq = gu.host(gu.quantize_weights("q80", x))
    assert np.array_equal(wq, oracle.quantize_q80(x))


# ---------------------------------------------------------------- weights --
@pytest.mark.parametrize("wtype", ALL)
@pytest.mark.parametrize("sigma", [0.02, 0.002, 1.0, 40.0])
def test_quantize_weights_bitexact(wtype, sigma):
    _say("quantize_weights", wtype, sigma)
    rng = np.random.default_rng(int(sigma * 1000))
    w = (rng.standard_normal((37, 768)) * sigma).astype(np.float32)
    w[1] = np.abs(w[1])
    w[2] = -np.abs(w[2])
    w[3, :256] = 0.0
    w[4, 32:64] = np.float32(-0.25 * sigma)
    w[5, 0:16] = np.float32(0.0)
    w[5, 16] = np.float32(-0.0)
    w[6, 0:32] = np.float32(0.5 * sigma)           # equal magnitudes: the first one decides
    w[6, 40] = np.float32(-3 * sigma)
    w[6, 41] = np.float32(3 * sigma)
    w[7, 0] = np.float32(8 * sigma)                # the opposite extreme gets clipped (Q4_0)
    w[7, 1:32] = np.float32(-7.9 * sigma)
    got = gu.host(gu.quantize_weights(wtype, w))
    assert np.array_equal(got, _quant(wtype, w))


@pytest.mark.parametrize("wtype", ALL)
def test_quantize_weights_rows_pieces(wtype):
    """Row ranges quantized in pieces, in any order, give the one-call tensor byte for byte,
    and one piece writes only its own rows' bytes in every plane."""
    import torch
    import block_quantized_weight_act_amd as qg
    rows, cols = 37, 768
    _say("quantize_weights_rows", wtype, rows, cols)
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((rows, cols)) * 0.03).astype(np.float32)
    ref = _quant(wtype, w)
    out = torch.full((qg.qgemv_weight_bytes(wtype, rows, cols),), 0xAB, dtype=torch.uint8,
                     device=gu.DEV)
    for r0, r1 in [(6, 37), (0, 5), (5, 6)]:
        qg.qgemv_quantize_weights_rows(wtype, gu.dev(w[r0:r1]), out, rows, cols, r0, r1 - r0)
    assert np.array_equal(gu.host(out), ref)
    out.fill_(0xAB)
    qg.qgemv_quantize_weights_rows(wtype, gu.dev(w[9:14]), out, rows, cols, 9, 5)
    got_planes = oracle.planes(wtype, gu.host(out), rows, cols)
    for got, want in zip(got_planes, oracle.planes(wtype, ref, rows, cols)):
        assert np.array_equal(got[9:14], want[9:14])
        assert (got[:9] == 0xAB).all() and (got[14:] == 0xAB).all()


# ---------------------------------------------------------------- GEMV ------
def _check_gemv(wtype, wbuf, rows, cols, x, plan=None, debug=True):
    nvec = x.shape[0]
    rq, rd = oracle.quantize_act(x)
    xq, xd = gu.quantize_act(x)
    assert np.array_equal(gu.host(xq), rq)
    ref = oracle.gemv(wtype, wbuf, rows, cols, rq, rd, partials=debug)
    wt = gu.dev(wbuf)
    y = gu.gemv(wtype, wt, xq, xd, rows, cols, nvec, plan=plan)
    gu.assert_within_bound(y, ref)
    if debug:
        P, S = gu.partials(wtype, wt, xq, xd, rows, cols, nvec)
        assert np.array_equal(P, ref["P"])
        assert np.array_equal(S, oracle.block_sums(rq))
    return y, ref


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_parity_full_size(name):
    """Each decode workload at its full size: the GPU-quantized weights equal the oracle's
    bytes, y is inside the bound for every row and vector, P and S are bit-exact."""
    wl = synth.WORKLOADS[name]
    _say("workload", name, wl.rows, wl.cols, wl.nvec)
    x = wl.activations()
    chunk = 16384
    parts = []
    for r0 in range(0, wl.rows, chunk):
        r1 = min(wl.rows, r0 + chunk)
        w = wl.weight_block(r0, r1)
        ref = _quant(wl.wtype, w)
        got = gu.host(gu.quantize_weights(wl.wtype, w))
        assert np.array_equal(got, ref), "weight bytes differ in rows %d..%d" % (r0, r1)
        parts.append(ref)
    wbuf = oracle.concat_rows(wl.wtype, [(p, min(chunk, wl.rows - i * chunk))
                                         for i, p in enumerate(parts)], wl.cols)
    _check_gemv(wl.wtype, wbuf, wl.rows, wl.cols, x)


@pytest.mark.parametrize("wtype", ["q4k", "q6k"])
@pytest.mark.parametrize("rows,cols,nvec", [(1, 256, 1), (3, 512, 1), (17, 768, 2), (100, 1280, 3),
                                            (257, 2304, 1), (64, 8448, 1), (33, 256 * 33, 2),
                                            (5, 1536, 8), (999, 1024, 5)])
def test_ragged_shapes(wtype, rows, cols, nvec):
    _say("ragged", wtype, rows, cols, nvec)
    rng = np.random.default_rng(rows * 7 + cols + nvec)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    wbuf = oracle.quantize_q4k(w) if wtype == "q4k" else oracle.quantize_q6k(w, negate_scales=True)
    x = rng.standard_normal((nvec, cols)).astype(np.float32)
    _check_gemv(wtype, wbuf, rows, cols, x)


@pytest.mark.parametrize("wtype", ["q40", "q80"])
@pytest.mark.parametrize("rows,cols,nvec", [(1, 32, 1), (3, 96, 1), (17, 800, 2), (100, 1056, 3),
                                            (64, 8224, 1), (5, 1504, 8), (999, 224, 5)])
def test_ragged_shapes_32_weight_blocks(wtype, rows, cols, nvec):
    """Q4_0 / Q8_0 on widths that are multiples of 32 but not of 256 (8224: split columns)."""
    _say("ragged32", wtype, rows, cols, nvec)
    rng = np.random.default_rng(rows * 5 + cols + nvec)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    x = rng.standard_normal((nvec, cols)).astype(np.float32)
    _check_gemv(wtype, _quant(wtype, w), rows, cols, x)


PLANS = [dict(lanes_per_row=t, chunks_per_lane=nc, waves_per_block=wv, blocks=b)
         for t, nc, wv, b in [(8, 1, 1, 1), (8, 4, 4, 3), (16, 1, 2, 7), (16, 3, 4, 64),
                              (32, 2, 4, 5), (64, 1, 4, 100), (64, 4, 1, 2), (64, 2, 3, 1000),
                              (32, 2, 8, 3), (64, 3, 8, 9), (64, 1, 6, 40)]]


@pytest.mark.parametrize("plan", PLANS, ids=lambda p: "T%d_NC%d_W%d_B%d" % (
    p["lanes_per_row"], p["chunks_per_lane"], p["waves_per_block"], p["blocks"]))
@pytest.mark.parametrize("wtype", ALL)
def test_explicit_plans_and_splits(wtype, plan):
    """Every lane geometry, including column splits with the two-pass reduce."""
    rows, cols, nvec = 203, 2560, 2
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    wbuf = _quant(wtype, w)
    x = rng.standard_normal((nvec, cols)).astype(np.float32)
    nv = nvec if nvec * plan["chunks_per_lane"] <= 8 else 1
    _check_gemv(wtype, wbuf, rows, cols, x[:nv], plan=plan, debug=False)


@pytest.mark.parametrize("wtype", ALL)
def test_special_inputs(wtype):
    rows, cols = 64, 1024
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    wbuf = _quant(wtype, w, negate=True)
    what = oracle.dequantize(wtype, wbuf, rows, cols)
    # zero activation: y is exactly zero
    y, _ = _check_gemv(wtype, wbuf, rows, cols, np.zeros((1, cols), np.float32))
    assert np.all(y == 0)
    # one-hot activation: column extraction, y = w[:, k] * x_k; the Q4_K term of a small
    # dequantized weight cancels between its scale and min parts
    for k in list(range(0, cols, 13)) + [31, 32, cols - 1]:
        x = np.zeros((1, cols), np.float32)
        x[0, k] = -2.5
        y, ref = _check_gemv(wtype, wbuf, rows, cols, x)
        xq, xd = oracle.quantize_act(x)
        assert np.allclose(y[0], what[:, k] * (float(xd[0, k // 32]) * int(xq[0, k])),
                           rtol=1e-6, atol=0)
    # constant activation
    _check_gemv(wtype, wbuf, rows, cols, np.full((2, cols), 0.7, np.float32))
    # zero weights: y is exactly zero
    zbuf = _quant(wtype, np.zeros((rows, cols), np.float32))
    y, _ = _check_gemv(wtype, zbuf, rows, cols, rng.standard_normal((1, cols)).astype(np.float32))
    assert np.all(y == 0)


@pytest.mark.parametrize("sigma", [0.002, 30.0])
@pytest.mark.parametrize("wtype", ALL)
def test_scale_extremes(wtype, sigma):
    """Subnormal fp16 super-scales (sigma 0.002) and large ones (sigma 30)."""
    rows, cols = 128, 2048
    w = synth.normal_f32(77, 0, rows * cols, sigma).reshape(rows, cols)
    wbuf = _quant(wtype, w, negate=True)
    x = synth.normal_f32(78, 0, 2 * cols, 1.0).reshape(2, cols)
    _check_gemv(wtype, wbuf, rows, cols, x)


def test_integer_extremes():
    cols = 512
    blk = oracle.q4k_pack_block(0x3C00, 0x3C00, np.full(8, 63, np.uint8), np.full(8, 63, np.uint8),
                                np.full(256, 15, np.uint8))
    wbuf = oracle.q4k_tensor([blk] * (2 * 5))
    _check_gemv("q4k", wbuf, 5, cols, np.full((1, cols), 3.0, np.float32))
    body = oracle.q6k_pack_block(np.full(16, -128, np.int8), np.zeros(256, np.uint8))
    t6 = oracle.q6k_tensor([body] * (2 * 5), [0x3C00] * (2 * 5))
    _check_gemv("q6k", t6, 5, cols, np.full((1, cols), -3.0, np.float32))
    # Q8_0: codes 127 against 127 (P = 516128); Q4_0: codes 0 and 15 against -127
    img = oracle.q80_pack_block(np.float32(1.0), np.full(32, 127, np.int8))
    _check_gemv("q80", oracle.q32_tensor("q80", [img] * (16 * 5)), 5, cols,
                np.full((1, cols), 3.0, np.float32))
    img0 = oracle.q40_pack_block(0x3C00, np.zeros(32, np.uint8))
    img15 = oracle.q40_pack_block(0x3C00, np.full(32, 15, np.uint8))
    _check_gemv("q40", oracle.q32_tensor("q40", [img0, img15] * (8 * 5)), 5, cols,
                np.full((1, cols), -3.0, np.float32))


@pytest.mark.parametrize("wtype", ALL)
def test_determinism_permutation_and_batch(wtype):
    rows, cols = 300, 3072
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    wbuf = _quant(wtype, w)
    x = rng.standard_normal((1, cols)).astype(np.float32)
    xq, xd = gu.quantize_act(x)
    wt = gu.dev(wbuf)
    y1 = gu.gemv(wtype, wt, xq, xd, rows, cols, 1)
    y2 = gu.gemv(wtype, wt, xq, xd, rows, cols, 1)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))      # run-to-run identical
    perm = rng.permutation(rows)
    wp = _quant(wtype, w[perm])
    yp = gu.gemv(wtype, gu.dev(wp), xq, xd, rows, cols, 1)
    assert np.array_equal(yp[0].view(np.uint32), y1[0, perm].view(np.uint32))
    # a batch of identical vectors gives identical rows
    xb = np.repeat(x, 6, axis=0)
    xqb, xdb = gu.quantize_act(xb)
    yb = gu.gemv(wtype, wt, xqb, xdb, rows, cols, 6)
    for v in range(1, 6):
        assert np.array_equal(yb[v].view(np.uint32), yb[0].view(np.uint32))


def test_workspace_required_when_split():
    import block_quantized_weight_act_amd as qg
    rows, cols = 64, 4096
    plan = dict(lanes_per_row=16, chunks_per_lane=1, waves_per_block=4, blocks=4)
    assert qg.qgemv_plan_workspace_bytes(plan, rows, cols, 1) == 8 * rows * 4
    w = gu.dev(np.zeros(qg.qgemv_weight_bytes("q4k", rows, cols), np.uint8))
    xq, xd = gu.quantize_act(np.ones((1, cols), np.float32))
    import torch
    y = torch.empty((1, rows), dtype=torch.float32, device=gu.DEV)
    with pytest.raises(qg.QgemvError) as e:
        qg.qgemv_batch_plan("q4k", w, xq, xd, y, rows, cols, 1, plan)
    assert e.value.status == 3


@pytest.mark.parametrize("wtype,rows,cols,nvec", [
    ("q4k", 262144, 1536, 1), ("q4k", 8192, 2048, 1), ("q6k", 2048, 8192, 1),
    ("q4k", 16384, 2048, 8), ("q4k", 512, 512, 1), ("q6k", 333, 8448, 3), ("q4k", 77, 8448, 2),
    ("q4k", 1536, 6144, 1), ("q4k", 8192, 2048, 2), ("q6k", 2048, 8192, 2),
    ("q40", 4099, 1504, 1), ("q80", 1000, 2080, 2), ("q40", 300, 8224, 3), ("q80", 64, 96, 8),
])
def test_fused_quantize_and_gemv(wtype, rows, cols, nvec):
    """qgemv_fused: its codes and scales are the oracle's bit for bit, its y lies within the
    oracle's bound, and its y is bit-identical to quantize-then-GEMV with the same plan,
    including shapes whose plan splits the columns. With code outputs the library may take
    the two-launch route; without them it always runs the one-launch kernel (each workgroup
    quantizing its own slice). Past 16384 rows the weights repeat a 16384-row block of the
    oracle's tensor, so the oracle's y for that block, repeated, is the reference for every
    row."""
    import torch
    import block_quantized_weight_act_amd as qg
    _say("fused", wtype, rows, cols, nvec)
    rng = np.random.default_rng(rows + cols + nvec)
    x = (rng.standard_normal((nvec, cols)) * rng.choice([1e-3, 1.0, 40.0], size=(nvec, 1))).astype(np.float32)
    x[0, 32:64] = 0.0
    unique = min(rows, 16384)
    assert rows % unique == 0
    wbuf_u = _quant(wtype, (rng.standard_normal((unique, cols)) * 0.02).astype(np.float32))
    wbuf = wbuf_u if unique == rows else oracle.concat_rows(
        wtype, [(wbuf_u, unique)] * (rows // unique), cols)
    rq, rd = oracle.quantize_act(x)
    ref_u = oracle.gemv(wtype, wbuf_u, unique, cols, rq, rd)
    ref = {k: np.tile(ref_u[k], (1, rows // unique)) for k in ("y", "bound")}
    w = gu.dev(wbuf)
    xt = gu.dev(x)
    xq, xd = gu.quantize_act(x)
    y_two = gu.gemv(wtype, w, xq, xd, rows, cols, nvec)
    y = torch.full((nvec, rows), float("nan"), dtype=torch.float32, device=gu.DEV)
    xq_out = torch.zeros((nvec, cols), dtype=torch.int8, device=gu.DEV)
    xd_out = torch.zeros((nvec, cols // 32), dtype=torch.float32, device=gu.DEV)
    nbytes = qg.qgemv_workspace_bytes(wtype, rows, cols, nvec)
    ws = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=gu.DEV) if nbytes else None
    qg.qgemv_fused(wtype, w, xt, y, rows, cols, nvec, xq_out=xq_out, xd_out=xd_out, workspace=ws)
    y_fused = gu.host(y)
    gu.assert_within_bound(y_fused, ref)
    assert np.array_equal(y_fused.view(np.uint32), y_two.view(np.uint32))
    assert np.array_equal(gu.host(xq_out), rq)
    assert np.array_equal(gu.host(xd_out).view(np.uint32), rd.view(np.uint32))
    y2 = torch.full_like(y, float("nan"))
    qg.qgemv_fused(wtype, w, xt, y2, rows, cols, nvec, workspace=ws)      # without code outputs
    y_one = gu.host(y2)
    gu.assert_within_bound(y_one, ref)
    assert np.array_equal(y_one.view(np.uint32), y_two.view(np.uint32))


@pytest.mark.parametrize("wtype", ALL)
@pytest.mark.parametrize("rows,cols,nvec", [(37, 16384, 1), (200, 12288, 2), (91, 8192, 3),
                                            (64, 4096, 5), (19, 4096, 8)])
def test_split_inside_workgroup_matches_two_pass(wtype, rows, cols, nvec):
    """Rows wider than one pass (two column chunks): from codes the column split runs inside
    the workgroup (the chunks' sums added in LDS); the one-launch fused form without code
    outputs does the same after its workgroup quantized both chunks into LDS. Both add the
    chunks in ascending order, so y must agree bit for bit, and lie within the oracle's
    bound."""
    import torch
    import block_quantized_weight_act_amd as qg
    _say("split-in-workgroup", wtype, rows, cols, nvec)
    plan = qg.qgemv_plan_for(wtype, rows, cols, nvec)
    assert plan["lanes_per_row"] == 64 and plan["splits"] == 2, plan   # 3+ vectors: reduce-scatter
    assert qg.qgemv_route(wtype, rows, cols, nvec) == "vector"
    rng = np.random.default_rng(rows + cols + nvec)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    x = rng.standard_normal((nvec, cols)).astype(np.float32)
    wbuf = _quant(wtype, w)
    wd = gu.dev(wbuf)
    xq, xd = gu.quantize_act(x)
    nbytes = qg.qgemv_workspace_bytes(wtype, rows, cols, nvec)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=gu.DEV)
    y_in = torch.full((nvec, rows), float("nan"), dtype=torch.float32, device=gu.DEV)
    qg.qgemv_batch(wtype, wd, xq, xd, y_in, rows, cols, nvec, workspace=ws)
    y_two = torch.full_like(y_in, float("nan"))
    qg.qgemv_fused(wtype, wd, gu.dev(x), y_two, rows, cols, nvec, workspace=ws)
    a, b = gu.host(y_in), gu.host(y_two)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    rq, rd = oracle.quantize_act(x)
    gu.assert_within_bound(a, oracle.gemv(wtype, wbuf, rows, cols, rq, rd))


@pytest.mark.parametrize("wtype", ALL)
@pytest.mark.parametrize("rows,cols,nvec", [(19, 16384, 8), (40, 65536, 1)])
def test_fused_split_beyond_lds_takes_two_passes(wtype, rows, cols, nvec):
    """Eight column chunks whose quantized slices (36 bytes per activation block per chunk:
    147 KB and 74 KB) do not fit in a workgroup's 64 KiB of LDS: the fused form without code
    outputs quantizes each chunk in its own workgroups, writes the chunks' sums to the
    workspace (filled with NaN first) and adds them in a second launch, in ascending order.
    From codes the eight chunks are split inside the workgroup. y agrees bit for bit and lies
    within the oracle's bound."""
    import torch
    import block_quantized_weight_act_amd as qg
    _say("fused split beyond LDS", wtype, rows, cols, nvec)
    plan = qg.qgemv_plan_for(wtype, rows, cols, nvec)
    assert plan["lanes_per_row"] == 64 and plan["splits"] == 8, plan
    assert qg.qgemv_route(wtype, rows, cols, nvec) == "vector"
    assert qg.qgemv_fused_launches(wtype, rows, cols, nvec, 0) == 1
    rng = np.random.default_rng(rows * 3 + cols + nvec)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    x = rng.standard_normal((nvec, cols)).astype(np.float32)
    wbuf = _quant(wtype, w)
    wd = gu.dev(wbuf)
    xq, xd = gu.quantize_act(x)
    nbytes = qg.qgemv_workspace_bytes(wtype, rows, cols, nvec)
    assert nbytes == 8 * nvec * rows * 4
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=gu.DEV)
    y_codes = torch.full((nvec, rows), float("nan"), dtype=torch.float32, device=gu.DEV)
    qg.qgemv_batch(wtype, wd, xq, xd, y_codes, rows, cols, nvec, workspace=ws)
    ws.fill_(0xFF)
    y_fused = torch.full_like(y_codes, float("nan"))
    qg.qgemv_fused(wtype, wd, gu.dev(x), y_fused, rows, cols, nvec, workspace=ws)
    a, b = gu.host(y_codes), gu.host(y_fused)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    rq, rd = oracle.quantize_act(x)
    gu.assert_within_bound(a, oracle.gemv(wtype, wbuf, rows, cols, rq, rd))
