"""GPU parity of the matrix-core path (Q4_K with 17..256 activation vectors) against the CPU
oracle, through the C-ABI: integer partials P and activation block sums S bit-exact (debug
form), every y within 1e-5 of sum_i |w_i| |x_i| of its row and vector. Shapes cover every
vector-tile count (1..3 tiles of 32 in one group; groups of 2 tiles beyond 96 vectors), ragged row tiles, column
splits (few rows) and one pass (many rows)."""

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.require_gpu()


def _say(*a):
    print("[mfma]", *a, flush=True)


def _check(wbuf, rows, cols, x, debug=True):
    import block_quantized_weight_act_amd as qg
    nvec = x.shape[0]
    rq, rd = oracle.quantize_act(x)
    xq, xd = gu.quantize_act(x)
    assert np.array_equal(gu.host(xq), rq)
    ref = oracle.gemv("q4k", wbuf, rows, cols, rq, rd, partials=debug)
    wt = gu.dev(wbuf)
    y = gu.gemv("q4k", wt, xq, xd, rows, cols, nvec)
    gu.assert_within_bound(y, ref)
    if debug:
        P, S = gu.partials("q4k", wt, xq, xd, rows, cols, nvec)
        assert np.array_equal(S, oracle.block_sums(rq))
        assert np.array_equal(P, ref["P"])
    return y, ref, wt, xq, xd


SHAPES = [
    # (rows, cols, nvec)
    (300, 512, 17),       # one tile of 32 vectors, 15 idle; ragged last row tile; split
    (257, 768, 33),       # two tiles
    (128, 2048, 64),      # one row tile, split over 8 super-blocks
    (1000, 1536, 100),    # two groups of two tiles (100 of 128)
    (131, 256, 128),      # one super-block: no split possible; two groups
    (64, 4096, 129),      # three vector groups (64 + 64 + 1)
    (513, 1024, 256),     # four full groups of 64
    (4100, 1536, 40),     # enough rows for one pass (no split)
    (37, 2560, 77),       # three tiles in one group, ragged everything
    (200, 1024, 96),      # three full tiles in one group
]


@pytest.mark.parametrize("rows,cols,nvec", SHAPES)
def test_parity(rows, cols, nvec):
    _say("shape", rows, cols, nvec)
    rng = np.random.default_rng(rows * 31 + cols + nvec)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    w[rng.integers(0, rows, size=max(1, rows // 50))] *= 10.0       # outlier rows
    x = (rng.standard_normal((nvec, cols)) *
         rng.choice([0.01, 1.0, 30.0], size=(nvec, 1))).astype(np.float32)
    x[nvec // 2] = 0.0                                               # a zero vector
    x[:, rng.integers(0, cols, size=cols // 8)] = 0.0                # zero columns
    _check(oracle.quantize_q4k(w), rows, cols, x)


def test_integer_extremes():
    """Largest codes and sub-scales against +-127 activations: P = +-60960 per block, the
    largest sc * q (945) in every operand."""
    rows, cols, nvec = 70, 512, 40
    blk = oracle.q4k_pack_block(0x3C00, 0x3C00, np.full(8, 63, np.uint8), np.full(8, 63, np.uint8),
                                np.full(256, 15, np.uint8))
    wbuf = oracle.q4k_tensor([blk] * (rows * 2))
    x = np.full((nvec, cols), 3.0, np.float32)
    x[1::2] = -3.0
    _, ref, *_ = _check(wbuf, rows, cols, x)
    assert np.abs(ref["P"]).max() == 60960


def test_deterministic_batch_rows_and_untouched_outside():
    """Run-to-run identical bits; identical vectors give identical rows of y; nothing outside
    y is written."""
    import torch
    import block_quantized_weight_act_amd as qg
    rows, cols = 515, 1024
    rng = np.random.default_rng(5)
    wt = gu.dev(oracle.quantize_q4k((rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)))
    x = rng.standard_normal((1, cols)).astype(np.float32)
    nvec = 70
    xq, xd = gu.quantize_act(np.repeat(x, nvec, axis=0))
    pool = torch.full((nvec * rows + 64,), 7.0, dtype=torch.float32, device=gu.DEV)
    y = pool[32:32 + nvec * rows].view(nvec, rows)
    nbytes = qg.qgemv_workspace_bytes("q4k", rows, cols, nvec)
    ws = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=gu.DEV)
    qg.qgemv_batch("q4k", wt, xq, xd, y, rows, cols, nvec, workspace=ws)
    first = gu.host(pool).copy()
    for _ in range(2):
        qg.qgemv_batch("q4k", wt, xq, xd, y, rows, cols, nvec, workspace=ws)
        assert np.array_equal(gu.host(pool).view(np.uint32), first.view(np.uint32))
    assert (first[:32] == 7.0).all() and (first[32 + nvec * rows:] == 7.0).all()
    yy = first[32:32 + nvec * rows].reshape(nvec, rows)
    for v in range(1, nvec):
        assert np.array_equal(yy[v].view(np.uint32), yy[0].view(np.uint32))


def test_workspace_and_limits():
    import torch
    import block_quantized_weight_act_amd as qg
    rows, cols, nvec = 256, 2048, 64          # few rows: the super-blocks are split
    assert qg.qgemv_workspace_bytes("q4k", rows, cols, nvec) > 0
    assert qg.qgemv_workspace_bytes("q4k", 65536, cols, nvec) == 8 * 2 * 18432   # tiles only
    w = torch.zeros(qg.qgemv_weight_bytes("q4k", rows, cols), dtype=torch.uint8, device=gu.DEV)
    xq = torch.zeros((257, cols), dtype=torch.int8, device=gu.DEV)
    xd = torch.zeros((257, cols // 32), dtype=torch.float32, device=gu.DEV)
    y = torch.zeros((257, rows), dtype=torch.float32, device=gu.DEV)
    with pytest.raises(qg.QgemvError):       # no workspace
        qg.qgemv_batch("q4k", w, xq, xd, y, rows, cols, nvec)
    with pytest.raises(qg.QgemvError):       # more vectors than the matrix-core path takes
        qg.qgemv_batch("q4k", w, xq, xd, y, rows, cols, 257,
                       workspace=torch.zeros(1 << 24, dtype=torch.uint8, device=gu.DEV))
    torch.cuda.synchronize()


def test_full_size_vocabulary_projection_sampled():
    """The 262144 x 1536 projection with 64 vectors (the launch the bench times): every output
    finite, sampled rows against the oracle's bound, integer partials of sampled rows exact."""
    import torch
    import block_quantized_weight_act_amd as qg
    import synth
    wl = synth.WORKLOADS["q4k_262144x1536"]
    rows, cols, nvec = wl.rows, wl.cols, 64
    _say("full size", rows, cols, nvec)
    w = torch.empty(qg.qgemv_weight_bytes("q4k", rows, cols), dtype=torch.uint8, device=gu.DEV)
    for r0 in range(0, rows, 32768):
        wf = gu.dev(wl.weight_block(r0, r0 + 32768))
        qg.qgemv_quantize_weights_rows("q4k", wf, w, rows, cols, r0, 32768)
        del wf
    x = np.stack([synth.normal_f32(9100 + v, 0, cols, 1.0) for v in range(nvec)])
    rq, rd = oracle.quantize_act(x)
    xq, xd = gu.quantize_act(x)
    y = torch.empty((nvec, rows), dtype=torch.float32, device=gu.DEV)
    nbytes = qg.qgemv_workspace_bytes("q4k", rows, cols, nvec)
    ws = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=gu.DEV)
    qg.qgemv_batch("q4k", w, xq, xd, y, rows, cols, nvec, workspace=ws)
    yh = gu.host(y)
    assert np.all(np.isfinite(yh))
    sample = np.unique(np.concatenate([np.arange(0, rows, 4099), wl.outlier_rows()[::50],
                                       [rows - 1]]))
    wbuf = oracle.quantize_q4k(wl.weight_rows(sample))
    ref = oracle.gemv("q4k", wbuf, sample.size, cols, rq, rd)
    gu.assert_within_bound(yh[:, sample], ref)


@pytest.mark.parametrize("rows,cols,nvec", [
    (40000, 1536, 25),    # one vector tile, 313 row tiles: 2 splits of 3 super-blocks (odd)
    (70000, 1280, 17),    # one vector tile, 547 row tiles: no split, 5 super-blocks (odd)
])
def test_odd_super_block_counts_sampled(rows, cols, nvec):
    """Many rows with an odd number of super-blocks per workgroup (the one-tile kernel keeps
    weights two super-blocks ahead and pads odd counts): sampled rows against the oracle."""
    import torch
    import block_quantized_weight_act_amd as qg
    _say("odd", rows, cols, nvec)
    rng = np.random.default_rng(rows + nvec)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    wbuf = oracle.quantize_q4k(w)
    x = rng.standard_normal((nvec, cols)).astype(np.float32)
    rq, rd = oracle.quantize_act(x)
    xq, xd = gu.quantize_act(x)
    y = gu.gemv("q4k", gu.dev(wbuf), xq, xd, rows, cols, nvec)
    sample = np.unique(np.concatenate([np.arange(0, rows, 97), np.arange(rows - 300, rows)]))
    sbuf = oracle.quantize_q4k(w[sample])
    ref = oracle.gemv("q4k", sbuf, sample.size, cols, rq, rd)
    gu.assert_within_bound(y[:, sample], ref)
    torch.cuda.synchronize()
