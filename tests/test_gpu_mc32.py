"""GPU parity of the integer matrix-core path for 9..256 activation vectors (Q8_0 and Q4_0: one
32 x 32 x 32 product per 32-weight block; Q6_K: one 32 x 32 x 16 product per 16-weight
sub-block) and for 1..8 Q8_0 and Q4_0 vectors (16 x 16 x 64 products over the halves of 4
blocks) against the CPU oracle, through the C ABI: integer partials P (per block, or per
Q6_K sub-block) and activation block sums S bit-exact (debug form), every y within 1e-5 of
sum_i |w_i| |x_i| of its row and vector. Shapes cover 1, 2 and 4 vector tiles of 32 per
workgroup, one and two vector groups, ragged row tiles, widths that are not a whole number of
4-block steps, column splits (few rows; for Q6_K splits that start in the middle of a
super-block) and one pass (many rows), the int32 extremes of every format, and the
262144 x 1536 vocabulary projection with 64 vectors (sampled rows); with 1..8 vectors, one to
four waves per workgroup, waves and splits that end inside their 16 blocks, the last split of
one block, one and two halves of 4 vectors, and workgroups that walk more than two row tiles."""

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
    print("[mc32]", *a, flush=True)


def _mc32(wtype, wt, xq, xd, rows, cols, nvec):
    """y of the matrix-core kernel itself (qgemv_batch_mc32), whichever route qgemv_batch
    takes for the shape."""
    import torch
    import block_quantized_weight_act_amd as qg
    y = torch.full((nvec, rows), float("nan"), dtype=torch.float32, device=gu.DEV)
    nbytes = qg.qgemv_mc32_workspace_bytes(wtype, rows, cols, nvec)
    ws = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=gu.DEV) if nbytes else None
    qg.qgemv_batch_mc32(wtype, wt, xq, xd, y, rows, cols, nvec, workspace=ws)
    return gu.host(y)


def _check(wtype, wbuf, rows, cols, x, debug=True):
    import block_quantized_weight_act_amd as qg
    nvec = x.shape[0]
    rq, rd = oracle.quantize_act(x)
    xq, xd = gu.quantize_act(x)
    assert np.array_equal(gu.host(xq), rq)
    ref = oracle.gemv(wtype, wbuf, rows, cols, rq, rd, partials=debug)
    wt = gu.dev(wbuf)
    y = _mc32(wtype, wt, xq, xd, rows, cols, nvec)
    gu.assert_within_bound(y, ref)
    # qgemv_batch: the same kernel (bit for bit) where it routes there, else the vector kernel
    # (on groups of 8 with more than 8 vectors), within the same bound
    route = qg.qgemv_route(wtype, rows, cols, nvec)
    assert route in (("mc32", "vector", "i8mc") if nvec <= 8 else ("mc32", "grouped", "i8mc"))
    yb = gu.gemv(wtype, wt, xq, xd, rows, cols, nvec)
    if route == "mc32":
        assert np.array_equal(yb.view(np.uint32), y.view(np.uint32))
    else:
        gu.assert_within_bound(yb, ref)
    if debug:
        # the kernel's own partials, and those of the route qgemv_debug_partials takes
        P, S = _mc32_partials(wtype, wt, xq, xd, rows, cols, nvec)
        assert np.array_equal(S, oracle.block_sums(rq))
        assert np.array_equal(P, ref["P"])
        P, S = gu.partials(wtype, wt, xq, xd, rows, cols, nvec)
        assert np.array_equal(S, oracle.block_sums(rq))
        assert np.array_equal(P, ref["P"])
    return y


def _mc32_partials(wtype, wt, xq, xd, rows, cols, nvec):
    import torch
    import block_quantized_weight_act_amd as qg
    nsub = cols // 16 if wtype == "q6k" else cols // 32
    P = torch.full((nvec, rows, nsub), -(2 ** 31), dtype=torch.int32, device=gu.DEV)
    S = torch.full((nvec, cols // 32), -(2 ** 31), dtype=torch.int32, device=gu.DEV)
    qg.qgemv_debug_partials_mc32(wtype, wt, xq, xd, P, S, rows, cols, nvec)
    return gu.host(P), gu.host(S)


SHAPES = [
    # (rows, cols, nvec)
    (300, 1056, 9),       # one tile of 32 vectors (23 idle), 33 blocks (a ragged step), split
    (257, 768, 33),       # two tiles
    (128, 2048, 64),      # one row tile, split
    (1000, 1536, 100),    # four tiles (100 of 128)
    (131, 32, 128),       # one block: no split possible
    (64, 4096, 129),      # two vector groups (128 + 1)
    (513, 1024, 256),     # two full groups of 128
    (4100, 1536, 40),     # enough rows for one pass (no split)
    (37, 2592, 77),       # three tiles, ragged everything
]


SHAPES_Q6K = [
    # (rows, cols, nvec): Q6_K rows are whole super-blocks of 256 columns
    (300, 1280, 9),       # 40 blocks over 10 splits of half a super-block each
    (257, 768, 33),
    (128, 2048, 64),
    (1000, 1536, 100),
    (131, 256, 128),      # one super-block: two steps
    (64, 4096, 129),
    (513, 1024, 256),
    (4100, 1536, 40),
    (37, 2560, 77),
    (2048, 8192, 64),     # the short, wide matrix with 64 vectors
]

SHAPES_FEW = [
    # (rows, cols, nvec): 1..8 Q8_0 / Q4_0 vectors
    (300, 1056, 3),       # 33 blocks: three waves, the third with one block; ragged row tiles
    (257, 768, 8),        # two waves, two halves of 4 vectors
    (128, 2048, 5),       # four full waves, one row tile pair
    (1000, 4096, 7),      # two splits of 64 blocks
    (131, 32, 1),         # one block, one wave
    (64, 8224, 4),        # 257 blocks: five splits of four waves, the last of one block
    (4100, 1536, 6),      # three waves, 257 row tiles
    (37, 2592, 2),        # 81 blocks: two splits of three waves, ragged
    (20000, 2048, 3),     # 1250 row tiles: workgroups walk more than two
    (20000, 1600, 8),     # 50 blocks over four waves, more than two tiles per workgroup
    (16384, 2048, 5),     # where qgemv_batch takes this kernel for Q4_0
]

SHAPES_FEW_Q6K = [
    # (rows, cols, nvec): 1..8 Q6_K vectors (rows of whole super-blocks)
    (300, 1280, 3),       # 40 blocks: three waves, the third with one super-block
    (257, 768, 8),        # two waves, the second with one super-block; two halves of 4 vectors
    (128, 2048, 5),       # four full waves
    (1000, 4096, 7),      # two splits
    (131, 256, 1),        # one super-block, one wave
    (64, 8448, 4),        # 264 blocks: five splits of four waves, the last of one super-block
    (4100, 1536, 6),      # three waves, 257 row tiles
    (20000, 2048, 3),     # workgroups walk more than two row tiles
    (20000, 1536, 8),
    (16384, 2048, 4),     # where qgemv_batch takes this kernel for Q4_K
]

SHAPES_MID = [
    # (rows, cols, nvec): 9..16 vectors on tensors of at least 16 Mi weights, where the
    # few-vector kernel takes 3 or 4 halves of 4 vectors (Q4_K: 9..12)
    (8192, 2048, 12),     # one split of four waves, three halves
    (4096, 4096, 16),     # two splits, four halves
    (2048, 8192, 10),     # four splits, three halves (two vectors idle)
    (16384, 1280, 9),     # 40 blocks: three waves, the last with one super-block
]

CASES = ([(w, *s) for w in ("q80", "q40") for s in SHAPES] + [("q6k", *s) for s in SHAPES_Q6K] +
         [(w, *s) for w in ("q80", "q40", "q6k", "q4k") for s in SHAPES_MID
          if not (w == "q4k" and s[2] > 12)] +
         [(w, *s) for w in ("q80", "q40") for s in SHAPES_FEW] +
         [(w, *s) for w in ("q6k", "q4k") for s in SHAPES_FEW_Q6K])


@pytest.mark.parametrize("wtype,rows,cols,nvec", CASES)
def test_parity(wtype, rows, cols, nvec):
    _say(wtype, rows, cols, nvec)
    rng = np.random.default_rng(rows * 31 + cols + nvec + ("q80", "q40", "q6k", "q4k").index(wtype))
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    w[0, :64] = 0.0                                     # zero weight blocks: exactly 0
    x = (rng.standard_normal((nvec, cols)) * rng.choice([1e-3, 1.0, 40.0], size=(nvec, 1))).astype(np.float32)
    x[0, 32:64] = 0.0
    _check(wtype, oracle.quantize(wtype, w), rows, cols, x)


def test_integer_extremes():
    rows, cols, nvec = 70, 256, 12
    img = oracle.q80_pack_block(np.float32(1.0), np.full(32, 127, np.int8))
    t80 = oracle.q32_tensor("q80", [img] * (rows * cols // 32))
    _check("q80", t80, rows, cols, np.full((nvec, cols), 3.0, np.float32))     # P = 516128
    img0 = oracle.q40_pack_block(0x3C00, np.zeros(32, np.uint8))
    img15 = oracle.q40_pack_block(0x3C00, np.full(32, 15, np.uint8))
    t40 = oracle.q32_tensor("q40", [img0, img15] * (rows * cols // 64))
    _check("q40", t40, rows, cols, np.full((nvec, cols), -3.0, np.float32))    # P = +-32512
    # Q6_K: codes 0 and 63 (q - 32 = -32, 31) with sub-scales -128 and 127 against codes -127:
    # P = 65024 and -62992, sc0 P0 + sc1 P1 = -16646144 (just under 2^24 in magnitude)
    lo = oracle.q6k_pack_block(np.full(16, -128, np.int8), np.zeros(256, np.uint8))
    hi = oracle.q6k_pack_block(np.array([127, -128] * 8, np.int8),
                               np.array(([63] * 16 + [0] * 16) * 8, np.uint8))
    nsb = rows * cols // 256
    t6 = oracle.q6k_tensor([lo, hi] * (nsb // 2), [0x3C00, 0x0400] * (nsb // 2))
    _check("q6k", t6, rows, cols, np.full((nvec, cols), -3.0, np.float32))


def _random_few_cases(n=24, seed=20261202):
    """Seeded random shapes for the few-vector kernel: every format, 1..8 vectors, rows 1..3000,
    widths from one block to a few splits (whole super-blocks for Q4_K and Q6_K)."""
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        wtype = ("q80", "q40", "q6k", "q4k")[k % 4]
        unit = 256 if wtype in ("q4k", "q6k") else 32
        cols = unit * int(rng.integers(1, 9000 // unit + 1))
        rows = int(rng.integers(1, 3001))
        nvec = int(rng.integers(1, 9))
        cases.append((wtype, rows, cols, nvec))
    return cases


@pytest.mark.parametrize("wtype,rows,cols,nvec", _random_few_cases())
def test_few_vectors_random_shapes(wtype, rows, cols, nvec):
    """The few-vector kernel itself (qgemv_batch_mc32 / qgemv_debug_partials_mc32) on seeded
    random shapes: P and S bit-exact, y within the bound."""
    _say("random", wtype, rows, cols, nvec)
    rng = np.random.default_rng(rows * 13 + cols * 7 + nvec)
    w = (rng.standard_normal((rows, cols)) * rng.choice([0.002, 0.02, 0.5])).astype(np.float32)
    x = (rng.standard_normal((nvec, cols)) * rng.choice([1e-3, 1.0, 40.0], size=(nvec, 1))).astype(np.float32)
    _check(wtype, oracle.quantize(wtype, w), rows, cols, x)


def test_fused_with_code_outputs_takes_the_matrix_cores():
    """qgemv_fused with code outputs on a shape qgemv_batch runs on the few-vector matrix-core
    kernel: two launches, the oracle's codes and scales, and qgemv_batch's y bit for bit."""
    import torch
    import block_quantized_weight_act_amd as qg
    rows, cols, nvec = 16384, 2048, 6
    assert qg.qgemv_route("q40", rows, cols, nvec) == "mc32"
    assert qg.qgemv_fused_launches("q40", rows, cols, nvec, True) == 2
    rng = np.random.default_rng(17)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    x = (rng.standard_normal((nvec, cols)) * 2.0).astype(np.float32)
    wbuf = oracle.quantize("q40", w)
    rq, rd = oracle.quantize_act(x)
    wt = gu.dev(wbuf)
    xq = torch.empty((nvec, cols), dtype=torch.int8, device=gu.DEV)
    xd = torch.empty((nvec, cols // 32), dtype=torch.float32, device=gu.DEV)
    y = torch.full((nvec, rows), float("nan"), dtype=torch.float32, device=gu.DEV)
    nbytes = qg.qgemv_workspace_bytes("q40", rows, cols, nvec)
    ws = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=gu.DEV) if nbytes else None
    qg.qgemv_fused("q40", wt, gu.dev(x), y, rows, cols, nvec, xq_out=xq, xd_out=xd, workspace=ws)
    assert np.array_equal(gu.host(xq), rq)
    assert np.array_equal(gu.host(xd).view(np.uint32), rd.view(np.uint32))
    yb = gu.gemv("q40", wt, xq, xd, rows, cols, nvec)
    assert np.array_equal(gu.host(y).view(np.uint32), yb.view(np.uint32))
    gu.assert_within_bound(gu.host(y), oracle.gemv("q40", wbuf, rows, cols, rq, rd))


def test_integer_extremes_few_vectors():
    rows, cols, nvec = 70, 256, 8
    img = oracle.q80_pack_block(np.float32(1.0), np.full(32, -127, np.int8))
    t80 = oracle.q32_tensor("q80", [img] * (rows * cols // 32))
    _check("q80", t80, rows, cols, np.full((nvec, cols), 3.0, np.float32))     # P = -516128
    img0 = oracle.q40_pack_block(0x3C00, np.zeros(32, np.uint8))
    img15 = oracle.q40_pack_block(0x3C00, np.full(32, 15, np.uint8))
    t40 = oracle.q32_tensor("q40", [img15, img0] * (rows * cols // 64))
    _check("q40", t40, rows, cols, np.full((nvec, cols), -3.0, np.float32))    # P = -28448, 32512


def test_zero_weights_give_exact_zero():
    rows, cols, nvec = 96, 512, 20
    x = np.random.default_rng(3).standard_normal((nvec, cols)).astype(np.float32)
    for wtype in ("q80", "q40", "q6k"):
        y = _check(wtype, oracle.quantize(wtype, np.zeros((rows, cols), np.float32)), rows, cols, x,
                   debug=False)
        assert np.all(y == 0)
    for wtype in ("q80", "q40"):
        y = _check(wtype, oracle.quantize(wtype, np.zeros((rows, cols), np.float32)), rows, cols,
                   x[:6], debug=False)
        assert np.all(y == 0)


@pytest.mark.parametrize("wtype", ["q80", "q6k"])
def test_vocabulary_projection_64_vectors_sampled(wtype):
    """262144 x 1536 with 64 vectors, the workloads the many-vector bench times: the weights
    are the oracle's tensor (built in row pieces), the product runs whole on the GPU, and 4096
    evenly spaced rows are checked against the oracle."""
    import torch
    import block_quantized_weight_act_amd as qg
    wl = synth.WORKLOADS["%s_262144x1536" % wtype]
    rows, cols, nvec = wl.rows, wl.cols, 64
    _say("vocabulary projection", wtype, rows, cols, nvec)
    chunk = 32768
    parts = [(oracle.quantize(wtype, wl.weight_block(r0, min(rows, r0 + chunk))),
              min(chunk, rows - r0)) for r0 in range(0, rows, chunk)]
    wbuf = oracle.concat_rows(wtype, parts, cols)
    x = np.stack([synth.normal_f32(wl.seed_x + v, 0, cols, 1.0) for v in range(nvec)])
    rq, rd = oracle.quantize_act(x)
    xq, xd = gu.dev(rq), gu.dev(rd)
    y = torch.full((nvec, rows), float("nan"), dtype=torch.float32, device=gu.DEV)
    nbytes = qg.qgemv_workspace_bytes(wtype, rows, cols, nvec)
    ws = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=gu.DEV) if nbytes else None
    qg.qgemv_batch(wtype, gu.dev(wbuf), xq, xd, y, rows, cols, nvec, workspace=ws)
    sample = np.linspace(0, rows - 1, 4096).astype(np.int64)
    sampled = oracle.from_planes([p[sample] for p in oracle.planes(wtype, wbuf, rows, cols)])
    ref = oracle.gemv(wtype, sampled, sample.size, cols, rq, rd)
    gu.assert_within_bound(gu.host(y)[:, sample], ref)
