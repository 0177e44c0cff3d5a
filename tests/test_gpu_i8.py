"""GPU parity of the integer matrix-core path (Q4_K with 1..16 activation vectors,
v_mfma_i32_16x16x64_i8) against the CPU oracle, through the C-ABI: integer partials P and
activation block sums S bit-exact (debug form), every y within 1e-5 of sum_i |w_i| |x_i| of its
row and vector. Small shapes call the path directly (qgemv_*_i8mc) and cover every wave count
of a workgroup (1..4), waves with one of their two super-blocks past the split's end, one and
several column splits (workspace), ragged row tiles, one and many row tiles per workgroup and
the fused form (quantization inside the kernel); a full-size vocabulary projection with 8
vectors checks that qgemv_batch and qgemv_fused take this path by themselves."""

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.require_gpu()


def _say(*a):
    print("[i8]", *a, flush=True)


def _y(wt, xq, xd, rows, cols, nvec):
    import torch
    import block_quantized_weight_act_amd as qg
    y = torch.full((nvec, rows), float("nan"), dtype=torch.float32, device=gu.DEV)
    nbytes = qg.qgemv_i8mc_workspace_bytes(rows, cols, nvec)
    ws = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=gu.DEV) if nbytes else None
    qg.qgemv_batch_i8mc(wt, xq, xd, y, rows, cols, nvec, workspace=ws)
    return gu.host(y)


def _partials(wt, xq, xd, rows, cols, nvec):
    import torch
    import block_quantized_weight_act_amd as qg
    P = torch.full((nvec, rows, cols // 32), -(2 ** 31), dtype=torch.int32, device=gu.DEV)
    S = torch.full((nvec, cols // 32), -(2 ** 31), dtype=torch.int32, device=gu.DEV)
    qg.qgemv_debug_partials_i8mc(wt, xq, xd, P, S, rows, cols, nvec)
    return gu.host(P), gu.host(S)


def _inputs(rows, cols, nvec, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    w[rng.integers(0, rows, size=max(1, rows // 50))] *= 10.0       # outlier rows
    x = (rng.standard_normal((nvec, cols)) *
         rng.choice([0.01, 1.0, 30.0], size=(nvec, 1))).astype(np.float32)
    x[nvec // 2] = 0.0                                               # a zero vector
    x[:, rng.integers(0, cols, size=cols // 8)] = 0.0                # zero columns
    return w, x


SHAPES = [
    # (rows, cols, nvec)
    (300, 512, 2),        # one wave, ragged last row tile
    (257, 768, 3),        # two waves, the second with one super-block
    (16, 2048, 8),        # one row tile, four waves
    (1000, 1536, 5),      # three waves
    (131, 256, 7),        # one super-block
    (64, 4096, 4),        # two column splits
    (513, 2304, 6),       # two splits of 6 and 3 super-blocks (a wave with none)
    (37, 6144, 8),        # three splits
    (4100, 2048, 8),      # many row tiles per workgroup
    (2000, 1024, 2),
    (777, 1280, 1),       # one vector
    # two groups of 8 vectors per launch
    (300, 512, 9),
    (1000, 1536, 12),
    (4100, 2048, 16),
    (513, 2304, 13),      # two splits, a wave with no super-block
    (37, 6144, 16),
]


@pytest.mark.parametrize("rows,cols,nvec", SHAPES)
def test_parity(rows, cols, nvec):
    _say("shape", rows, cols, nvec)
    w, x = _inputs(rows, cols, nvec, rows * 31 + cols + nvec)
    wbuf = oracle.quantize_q4k(w)
    rq, rd = oracle.quantize_act(x)
    xq, xd = gu.quantize_act(x)
    assert np.array_equal(gu.host(xq), rq)
    ref = oracle.gemv("q4k", wbuf, rows, cols, rq, rd, partials=True)
    wt = gu.dev(wbuf)
    gu.assert_within_bound(_y(wt, xq, xd, rows, cols, nvec), ref)
    P, S = _partials(wt, xq, xd, rows, cols, nvec)
    assert np.array_equal(S, oracle.block_sums(rq))
    assert np.array_equal(P, ref["P"])


def test_integer_extremes():
    """Largest codes and sub-scales against +-127 activations: P = +-60960 per block."""
    rows, cols, nvec = 70, 512, 8
    blk = oracle.q4k_pack_block(0x3C00, 0x3C00, np.full(8, 63, np.uint8), np.full(8, 63, np.uint8),
                                np.full(256, 15, np.uint8))
    wbuf = oracle.q4k_tensor([blk] * (rows * 2))
    x = np.full((nvec, cols), 3.0, np.float32)
    x[1::2] = -3.0
    rq, rd = oracle.quantize_act(x)
    xq, xd = gu.quantize_act(x)
    ref = oracle.gemv("q4k", wbuf, rows, cols, rq, rd, partials=True)
    assert np.abs(ref["P"]).max() == 60960
    wt = gu.dev(wbuf)
    gu.assert_within_bound(_y(wt, xq, xd, rows, cols, nvec), ref)
    P, _ = _partials(wt, xq, xd, rows, cols, nvec)
    assert np.array_equal(P, ref["P"])


@pytest.mark.parametrize("nvec", [8, 16])
def test_deterministic_identical_vectors_and_untouched_outside(nvec):
    """Run-to-run identical bits; identical vectors give identical rows of y (each vector
    sits in different lanes); nothing outside y is written."""
    import torch
    import block_quantized_weight_act_amd as qg
    rows, cols = 515, 2048
    rng = np.random.default_rng(5)
    wt = gu.dev(oracle.quantize_q4k((rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)))
    x = rng.standard_normal((1, cols)).astype(np.float32)
    xq, xd = gu.quantize_act(np.repeat(x, nvec, axis=0))
    pool = torch.full((nvec * rows + 64,), 7.0, dtype=torch.float32, device=gu.DEV)
    y = pool[32:32 + nvec * rows].view(nvec, rows)
    qg.qgemv_batch_i8mc(wt, xq, xd, y, rows, cols, nvec)
    first = gu.host(pool).copy()
    for _ in range(2):
        qg.qgemv_batch_i8mc(wt, xq, xd, y, rows, cols, nvec)
        assert np.array_equal(gu.host(pool).view(np.uint32), first.view(np.uint32))
    assert (first[:32] == 7.0).all() and (first[32 + nvec * rows:] == 7.0).all()
    yy = first[32:32 + nvec * rows].reshape(nvec, rows)
    for v in range(1, nvec):
        assert np.array_equal(yy[v].view(np.uint32), yy[0].view(np.uint32))


@pytest.mark.parametrize("rows,cols,nvec", [(300, 1536, 8), (77, 8448, 2), (1000, 768, 5)])
def test_fused_matches_two_launches(rows, cols, nvec):
    """qgemv_fused_i8mc quantizes inside the kernel: its codes and scales are the oracle's
    bit for bit, and its y equals quantize-then-qgemv_batch_i8mc bit for bit, with and without
    code outputs."""
    import torch
    import block_quantized_weight_act_amd as qg
    _say("fused", rows, cols, nvec)
    w, x = _inputs(rows, cols, nvec, rows + cols + nvec)
    x[0, 32:64] = 0.0
    wbuf = oracle.quantize_q4k(w)
    wt = gu.dev(wbuf)
    xq, xd = gu.quantize_act(x)
    y_two = _y(wt, xq, xd, rows, cols, nvec)
    rq, rd = oracle.quantize_act(x)
    gu.assert_within_bound(y_two, oracle.gemv("q4k", wbuf, rows, cols, rq, rd))
    xt = gu.dev(x)
    nbytes = qg.qgemv_i8mc_workspace_bytes(rows, cols, nvec)
    ws = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=gu.DEV) if nbytes else None
    y = torch.full((nvec, rows), float("nan"), dtype=torch.float32, device=gu.DEV)
    xq_out = torch.zeros((nvec, cols), dtype=torch.int8, device=gu.DEV)
    xd_out = torch.zeros((nvec, cols // 32), dtype=torch.float32, device=gu.DEV)
    qg.qgemv_fused_i8mc(wt, xt, y, rows, cols, nvec, xq_out=xq_out, xd_out=xd_out, workspace=ws)
    assert np.array_equal(gu.host(y).view(np.uint32), y_two.view(np.uint32))
    assert np.array_equal(gu.host(xq_out), rq)
    assert np.array_equal(gu.host(xd_out).view(np.uint32), rd.view(np.uint32))
    y2 = torch.full_like(y, float("nan"))
    qg.qgemv_fused_i8mc(wt, xt, y2, rows, cols, nvec, workspace=ws)
    assert np.array_equal(gu.host(y2).view(np.uint32), y_two.view(np.uint32))


def test_workspace_for_split_rows():
    """Rows wider than one split (8 super-blocks) need the partial-sum workspace."""
    import torch
    import block_quantized_weight_act_amd as qg
    rows, cols, nvec = 64, 4096, 4
    assert qg.qgemv_i8mc_workspace_bytes(rows, cols, nvec) == 2 * nvec * rows * 4
    assert qg.qgemv_i8mc_workspace_bytes(rows, 2048, nvec) == 0
    w = torch.zeros(qg.qgemv_weight_bytes("q4k", rows, cols), dtype=torch.uint8, device=gu.DEV)
    xq = torch.zeros((nvec, cols), dtype=torch.int8, device=gu.DEV)
    xd = torch.zeros((nvec, cols // 32), dtype=torch.float32, device=gu.DEV)
    y = torch.zeros((nvec, rows), dtype=torch.float32, device=gu.DEV)
    with pytest.raises(qg.QgemvError) as e:
        qg.qgemv_batch_i8mc(w, xq, xd, y, rows, cols, nvec)
    assert e.value.status == 3
    torch.cuda.synchronize()


def test_full_size_batch8_sampled():
    """The 16384 x 2048 matrix with 8 vectors (multi-sequence decode) on this path: every
    output finite, sampled rows against the oracle's bound, their integer partials exact."""
    import torch
    import block_quantized_weight_act_amd as qg
    import synth
    wl = synth.WORKLOADS["q4k_16384x2048_b8"]
    rows, cols, nvec = wl.rows, wl.cols, wl.nvec
    _say("full size", rows, cols, nvec)
    w = torch.empty(qg.qgemv_weight_bytes("q4k", rows, cols), dtype=torch.uint8, device=gu.DEV)
    wf = gu.dev(wl.weight_block(0, rows))
    qg.qgemv_quantize_weights_rows("q4k", wf, w, rows, cols, 0, rows)
    del wf
    x = np.stack([synth.normal_f32(wl.seed_x + v, 0, cols, 1.0) for v in range(nvec)])
    rq, rd = oracle.quantize_act(x)
    xq, xd = gu.quantize_act(x)
    y = _y(w, xq, xd, rows, cols, nvec)
    assert np.all(np.isfinite(y))
    sample = np.unique(np.concatenate([np.arange(0, rows, 257), np.arange(rows - 40, rows)]))
    wbuf = oracle.quantize_q4k(wl.weight_rows(sample))
    ref = oracle.gemv("q4k", wbuf, sample.size, cols, rq, rd, partials=True)
    gu.assert_within_bound(y[:, sample], ref)
    P, _ = _partials(w, xq, xd, rows, cols, nvec)
    assert np.array_equal(P[:, sample], ref["P"])


def test_vocabulary_projection_routes_here():
    """262144 x 1536 (about 216 MiB of Q4_K) with 8 vectors: qgemv_batch and qgemv_fused take
    the integer matrix-core path by themselves (bit-identical to qgemv_batch_i8mc), sampled
    rows within the oracle's bound, the fused codes the oracle's."""
    import torch
    import block_quantized_weight_act_amd as qg
    import synth
    wl = synth.WORKLOADS["q4k_262144x1536"]
    rows, cols, nvec = wl.rows, wl.cols, 8
    _say("vocabulary projection", rows, cols, nvec)
    w = torch.empty(qg.qgemv_weight_bytes("q4k", rows, cols), dtype=torch.uint8, device=gu.DEV)
    for r0 in range(0, rows, 32768):
        wf = gu.dev(wl.weight_block(r0, r0 + 32768))
        qg.qgemv_quantize_weights_rows("q4k", wf, w, rows, cols, r0, 32768)
        del wf
    x = np.stack([synth.normal_f32(9300 + v, 0, cols, 1.0) for v in range(nvec)])
    rq, rd = oracle.quantize_act(x)
    xq, xd = gu.quantize_act(x)
    y_i8 = _y(w, xq, xd, rows, cols, nvec)
    y = gu.gemv("q4k", w, xq, xd, rows, cols, nvec)
    assert np.array_equal(y.view(np.uint32), y_i8.view(np.uint32))
    yf = torch.full((nvec, rows), float("nan"), dtype=torch.float32, device=gu.DEV)
    xq_out = torch.zeros((nvec, cols), dtype=torch.int8, device=gu.DEV)
    xd_out = torch.zeros((nvec, cols // 32), dtype=torch.float32, device=gu.DEV)
    qg.qgemv_fused("q4k", w, gu.dev(x), yf, rows, cols, nvec, xq_out=xq_out, xd_out=xd_out)
    assert np.array_equal(gu.host(yf).view(np.uint32), y_i8.view(np.uint32))
    assert np.array_equal(gu.host(xq_out), rq)
    sample = np.unique(np.concatenate([np.arange(0, rows, 4099), wl.outlier_rows()[::50],
                                       [rows - 1]]))
    ref = oracle.gemv("q4k", oracle.quantize_q4k(wl.weight_rows(sample)), sample.size, cols, rq, rd)
    gu.assert_within_bound(y[:, sample], ref)
