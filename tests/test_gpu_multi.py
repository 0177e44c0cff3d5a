"""GPU parity of the multi-matrix product (several matrices sharing one activation, one launch)
against the CPU oracle, matrix by matrix, and against the one-matrix product with the same lane
geometry (bit for bit). Bars as in test_gpu_parity: codes and scales bit-exact, each y within
1e-5 of sum_i |w_i| |x_i| of its row. Rows wider than one pass of lanes (up to 65536 columns)
are split into column chunks inside the workgroup; their y is bit-identical to the one-matrix
product's split with the same geometry, from codes and fused (the fused form quantizes every
chunk of the row into LDS, or, where those slices do not fit, needs code outputs and runs
from them)."""

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.require_gpu()


def _say(*a):
    print("[multi]", *a, flush=True)


def multi_geometry(cols, nvec):
    """Lanes per row, chunks per lane and column chunks the library uses for a multi-matrix
    launch: the least idle lanes among the geometries that cover a row in one pass, more
    chunks per lane preferred (at most 3 with 2 vectors); for a wider row the least idle lanes
    with each further pass priced as 2% of them (15% from 5 vectors), among the geometries with
    at most a workgroup's waves of passes (the documented planner rules, restated here for the
    bit-identity check)."""
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
                    best, best_cost = (t, nc, passes), cost
        if best is not None:
            return best


def fused_slices_fit(nvec, t, nc, splits):
    """Whether a split row's fused form quantizes in LDS: the slices of every chunk (36 bytes
    per 32-column block) and the chunks' row sums within 64 KiB, with the launch's waves per
    workgroup (8 for a slice of >= 128 blocks, else 4, in sets of `splits`)."""
    if splits == 1:
        return True
    maxw = 8 if nvec * t * nc >= 128 else 4
    waves = splits * (maxw // splits)
    g = {1: 4, 2: 2}.get(nc, 1)
    return 36 * nvec * t * nc * splits + 4 * nvec * waves * g * (64 // t) <= 65536


CASES = [
    # (cols, nvec, [(wtype, rows), ...])
    (1536, 1, [("q4k", 300), ("q4k", 37), ("q6k", 129)]),      # attention-like Q, K, V
    (2048, 2, [("q6k", 1), ("q4k", 513), ("q6k", 64), ("q4k", 7)]),
    (2048, 8, [("q4k", 100), ("q6k", 33)]),
    (4096, 3, [("q4k", 17), ("q6k", 50)]),
    (8192, 1, [("q6k", 40), ("q4k", 9)]),
    (256, 1, [("q4k" if i % 2 else "q6k", i + 1) for i in range(8)]),   # eight matrices
    (768, 5, [("q6k", 3)]),                                               # one matrix
    (1536, 1, [("q4k", 100), ("q40", 65), ("q80", 33), ("q6k", 20)]),    # all four formats
    (800, 2, [("q40", 50), ("q80", 70)]),                                 # width not /256
    (96, 8, [("q80", 5), ("q40", 3)]),
    # rows wider than one pass: the column split inside the workgroup
    (16384, 1, [("q4k", 300), ("q6k", 65)]),                              # 2 chunks, one format each
    (8448, 1, [("q4k", 37), ("q40", 50), ("q80", 20), ("q6k", 5)]),       # 3 chunks of 96 blocks
    (6144, 5, [("q6k", 70), ("q4k", 33)]),                                # 3 chunks, 6 waves
    (12288, 3, [("q80", 100), ("q6k", 9)]),
    (16384, 8, [("q4k", 40), ("q4k", 3)]),                                # 8 chunks: codes needed
    (65536, 1, [("q6k", 20), ("q80", 3)]),                                # 8 chunks of 256 blocks
    (14336, 2, [("q4k", 1000)]),                                          # one matrix, 7 chunks
    (14336, 1, [("q6k", 2048), ("q4k", 64)]),     # the planner's 7 chunks of 64 exceed 4 waves
]


def _case_id(c):
    return "c%d_v%d_%s" % (c[0], c[1], "-".join("%s%d" % m for m in c[2]))


@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_multi_parity(case):
    import torch
    import block_quantized_weight_act_amd as qg
    cols, nvec, spec = case
    _say("multi", _case_id(case))
    rng = np.random.default_rng(cols * 7 + nvec + len(spec))
    x = rng.standard_normal((nvec, cols)).astype(np.float32)
    x[0, :32] = 0.0
    bufs = []
    for wtype, rows in spec:
        w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
        bufs.append(oracle.quantize(wtype, w))
    rq, rd = oracle.quantize_act(x)
    xq, xd = gu.quantize_act(x)
    assert np.array_equal(gu.host(xq), rq)
    ws = [gu.dev(b) for b in bufs]
    ys = [torch.full((nvec, rows), float("nan"), dtype=torch.float32, device=gu.DEV)
          for _, rows in spec]
    mats = [(wtype, w, rows, y) for (wtype, rows), w, y in zip(spec, ws, ys)]
    qg.qgemv_multi(mats, xq, xd, cols, nvec)
    got = [gu.host(y) for y in ys]
    t, nc = qg.qgemv_multi_geometry(cols, nvec)
    t0, nc0, splits = multi_geometry(cols, nvec)
    assert (t, nc) == (t0, nc0)
    plan = dict(lanes_per_row=t, chunks_per_lane=nc, waves_per_block=4, blocks=7)
    for (wtype, rows), buf, w, y in zip(spec, bufs, ws, got):
        ref = oracle.gemv(wtype, buf, rows, cols, rq, rd)
        gu.assert_within_bound(y, ref)
        single = gu.gemv(wtype, w, xq, xd, rows, cols, nvec, plan=plan)
        assert np.array_equal(y.view(np.uint32), single.view(np.uint32)), (wtype, rows)

    # the fused form: the same y bit for bit, with and without code outputs
    xt = gu.dev(x)
    fits = fused_slices_fit(nvec, t, nc, splits)
    for outs in (False, True):
        for y in ys:
            y.fill_(float("nan"))
        if not outs and not fits:
            with pytest.raises(qg.QgemvError):
                qg.qgemv_multi_fused(mats, xt, cols, nvec)
            assert all(torch.isnan(y).all() for y in ys)
            continue
        if outs:
            xq_out = torch.zeros((nvec, cols), dtype=torch.int8, device=gu.DEV)
            xd_out = torch.zeros((nvec, cols // 32), dtype=torch.float32, device=gu.DEV)
            qg.qgemv_multi_fused(mats, xt, cols, nvec, xq_out=xq_out, xd_out=xd_out)
            assert np.array_equal(gu.host(xq_out), rq)
            assert np.array_equal(gu.host(xd_out).view(np.uint32), rd.view(np.uint32))
        else:
            qg.qgemv_multi_fused(mats, xt, cols, nvec)
        for y, y0 in zip(ys, got):
            assert np.array_equal(gu.host(y).view(np.uint32), y0.view(np.uint32))


def test_multi_deterministic_and_untouched_outside():
    """Repeated launches give identical bits; nothing outside each y is written."""
    import torch
    import block_quantized_weight_act_amd as qg
    cols, nvec = 1536, 2
    rng = np.random.default_rng(3)
    x = rng.standard_normal((nvec, cols)).astype(np.float32)
    xq, xd = gu.quantize_act(x)
    spec = [("q4k", 65), ("q6k", 31)]
    ws = [gu.dev(oracle.quantize_q4k((rng.standard_normal((r, cols)) * 0.02).astype(np.float32))
                 if t == "q4k" else
                 oracle.quantize_q6k((rng.standard_normal((r, cols)) * 0.02).astype(np.float32)))
          for t, r in spec]
    # both outputs inside one guarded buffer, with gaps
    pool = torch.full((nvec * (65 + 31) + 96,), 123.0, dtype=torch.float32, device=gu.DEV)
    y0 = pool[32:32 + nvec * 65].view(nvec, 65)
    y1 = pool[64 + nvec * 65:64 + nvec * 65 + nvec * 31].view(nvec, 31)
    mats = [("q4k", ws[0], 65, y0), ("q6k", ws[1], 31, y1)]
    qg.qgemv_multi(mats, xq, xd, cols, nvec)
    first = gu.host(pool).copy()
    for _ in range(3):
        qg.qgemv_multi(mats, xq, xd, cols, nvec)
        assert np.array_equal(gu.host(pool).view(np.uint32), first.view(np.uint32))
    keep = np.ones(pool.numel(), bool)
    keep[32:32 + nvec * 65] = False
    keep[64 + nvec * 65:64 + nvec * 65 + nvec * 31] = False
    assert (first[keep] == 123.0).all()
