"""Replay of a captured decode step (qgemv_graph_*) against the same calls made directly and
against the CPU oracle.

A small decode step (two layers and a head; all four weight formats; multi-matrix, fused,
split-column and from-codes products) is recorded once. Each replay runs with new inputs
written into the recorded input buffers, with direct work and synchronizations between the
replays, and must give the outputs of the same calls made directly bit for bit; those lie
within the oracle's bound |y - y_ref| <= 1e-5 sum_i |w_i| |x_i| and their activation codes
are the oracle's bit for bit."""


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
    print("[graph]", *a, flush=True)


SMALL = synth.decode_step(
    "decode_small", 2, 256, 512, 64, 768,
    head=synth.Workload("decode_small.head", "q40", 1000, 256, 1, 1999, 2999),
    formats=("q4k", "q80", "q6k", "q4k", "q40", "q4k", "q6k"))


class Step:
    """Device buffers of one decode step and the library calls that make it. The down
    projections run from codes with a forced three-way column split (quantization, then the
    product with the split inside the workgroup: two launches, the workspace shared); the head
    is fused with code outputs."""

    def __init__(self, step):
        import torch
        import block_quantized_weight_act_amd as qg
        self.qg = qg
        self.items = []         # (kind, item, x, outputs, extra)
        self.launches = 0
        ws_bytes = 0
        for kind, item in step.products():
            parts = item.parts if kind == "multi" else (item,)
            cols, nvec = parts[0].cols, parts[0].nvec
            ws = []
            for p in parts:
                buf = oracle.quantize(p.wtype, p.weight_block(0, p.rows))
                ws.append((p, buf, gu.dev(buf)))
            x = torch.zeros((nvec, cols), dtype=torch.float32, device=gu.DEV)
            ys = [torch.zeros((nvec, p.rows), dtype=torch.float32, device=gu.DEV) for p in parts]
            extra = {}
            if kind == "multi":
                self.launches += 1
            elif p.name.endswith(".down"):
                plan = qg.qgemv_plan_for(p.wtype, p.rows, cols, nvec)
                plan.update(lanes_per_row=8, chunks_per_lane=1, blocks=16)   # 3 column chunks
                extra["plan"] = plan
                extra["xq"] = torch.zeros((nvec, cols), dtype=torch.int8, device=gu.DEV)
                extra["xd"] = torch.zeros((nvec, cols // 32), dtype=torch.float32, device=gu.DEV)
                need = qg.qgemv_plan_workspace_bytes(plan, p.rows, cols, nvec)
                assert need > 0
                ws_bytes = max(ws_bytes, need)
                self.launches += 2
            else:
                outs = p is step.head
                if outs:
                    extra["xq"] = torch.zeros((nvec, cols), dtype=torch.int8, device=gu.DEV)
                    extra["xd"] = torch.zeros((nvec, cols // 32), dtype=torch.float32,
                                              device=gu.DEV)
                ws_need = qg.qgemv_workspace_bytes(p.wtype, p.rows, cols, nvec)
                ws_bytes = max(ws_bytes, ws_need)
                self.launches += qg.qgemv_fused_launches(p.wtype, p.rows, cols, nvec, outs)
                self.launches += ws_need > 0
            self.items.append((kind, parts, ws, x, ys, extra))
        self.workspace = torch.zeros(max(16, ws_bytes), dtype=torch.uint8, device=gu.DEV)

    def run(self):
        """Enqueue the step's calls on the current stream."""
        qg = self.qg
        for kind, parts, ws, x, ys, extra in self.items:
            cols, nvec = parts[0].cols, parts[0].nvec
            if kind == "multi":
                mats = [(p.wtype, w, p.rows, y) for (p, _, w), y in zip(ws, ys)]
                qg.qgemv_multi_fused(mats, x, cols, nvec)
            elif "plan" in extra:
                p, _, w = ws[0]
                qg.qgemv_quantize_act(x, extra["xq"], extra["xd"], cols, nvec)
                qg.qgemv_batch_plan(p.wtype, w, extra["xq"], extra["xd"], ys[0], p.rows, cols,
                                    nvec, extra["plan"], workspace=self.workspace)
            else:
                p, _, w = ws[0]
                qg.qgemv_fused(p.wtype, w, x, ys[0], p.rows, cols, nvec, xq_out=extra.get("xq"),
                               xd_out=extra.get("xd"), workspace=self.workspace)

    def set_inputs(self, rep):
        """New seeded inputs (stream rep of each product's activation seed) into the buffers."""
        import torch
        xs = []
        for kind, parts, ws, x, ys, extra in self.items:
            nvec, cols = x.shape
            a = np.stack([synth.normal_f32(parts[0].seed_x + v + 7919 * rep, 0, cols, 1.0)
                          for v in range(nvec)])
            x.copy_(torch.from_numpy(a))
            xs.append(a)
        return xs

    def clear_outputs(self):
        for kind, parts, ws, x, ys, extra in self.items:
            for y in ys:
                y.fill_(float("nan"))
            for k in ("xq", "xd"):
                if k in extra:
                    extra[k].fill_(0)

    def outputs(self):
        out = []
        for kind, parts, ws, x, ys, extra in self.items:
            out += [gu.host(y).copy() for y in ys]
            out += [gu.host(extra[k]).copy() for k in ("xq", "xd") if k in extra]
        return out

    def check_oracle(self, xs, outs):
        i = 0
        for (kind, parts, ws, x, ys, extra), a in zip(self.items, xs):
            rq, rd = oracle.quantize_act(a)
            cols = parts[0].cols
            for p, buf, _ in ws:
                gu.assert_within_bound(outs[i], oracle.gemv(p.wtype, buf, p.rows, cols, rq, rd))
                i += 1
            if "xq" in extra:
                assert np.array_equal(outs[i], rq)
                assert np.array_equal(outs[i + 1].view(np.uint32), rd.view(np.uint32))
                i += 2


def _same_bits(a, b):
    assert len(a) == len(b)
    for k, (u, v) in enumerate(zip(a, b)):
        assert u.dtype == v.dtype and u.shape == v.shape, k
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), k


def test_graph_replays_match_direct_calls_and_oracle():
    import torch
    import block_quantized_weight_act_amd as qg
    _say("build small decode step")
    step = Step(SMALL)
    step.set_inputs(0)
    step.run()                      # direct calls once before the capture
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    _say("capture")
    with torch.cuda.stream(side):
        qg.qgemv_graph_begin()
        step.run()
        graph = qg.qgemv_graph_end()
    torch.cuda.synchronize()
    kernels, others = graph.nodes()
    assert (kernels, others) == (step.launches, 0)

    for rep in range(1, 5):
        _say("replay", rep)
        xs = step.set_inputs(rep)
        step.clear_outputs()
        graph.launch()
        torch.cuda.synchronize()
        replayed = step.outputs()
        step.clear_outputs()
        step.run()
        torch.cuda.synchronize()
        direct = step.outputs()
        _same_bits(replayed, direct)
        step.check_oracle(xs, replayed)
    # back-to-back replays on one stream, then once more checked
    xs = step.set_inputs(9)
    for _ in range(3):
        graph.launch()
    torch.cuda.synchronize()
    step.check_oracle(xs, step.outputs())
    graph.close()


MC_CASES = [("q4k", 16384, 2048, 8, "i8mc"), ("q4k", 16384, 2048, 14, "i8mc"),
            ("q4k", 4096, 1536, 40, "mc"), ("q80", 16384, 2048, 16, "mc32"),
            ("q6k", 16384, 2048, 32, "mc32"),
            # the few-vector kernel: Q4_0 with two column splits and the ordered reduce, Q4_K
            # with 4 vectors in one split
            ("q40", 16384, 4096, 8, "mc32"), ("q4k", 16384, 2048, 4, "mc32")]


def test_graph_replays_the_matrix_core_routes():
    """The routes qgemv_batch takes for several vectors (the integer matrix cores for Q4_K with
    8 and 14 vectors, the fp16 matrix cores with their staging pre-pass for 40, the 32-weight and
    Q6_K integer kernels with their splits and ordered reduce, the few-vector kernel for Q4_0 and
    Q4_K) recorded with the activation
    quantization into one graph: every replay, with new inputs and direct work between, gives
    the direct calls' outputs bit for bit, and those lie within the oracle's bound on sampled
    rows."""
    import torch
    import block_quantized_weight_act_amd as qg
    rng = np.random.default_rng(77)
    cases = []
    for wtype, rows, cols, nvec, route in MC_CASES:
        assert qg.qgemv_route(wtype, rows, cols, nvec) == route
        w = gu.quantize_weights(wtype, (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32))
        x = torch.zeros((nvec, cols), dtype=torch.float32, device=gu.DEV)
        xq = torch.zeros((nvec, cols), dtype=torch.int8, device=gu.DEV)
        xd = torch.zeros((nvec, cols // 32), dtype=torch.float32, device=gu.DEV)
        y = torch.zeros((nvec, rows), dtype=torch.float32, device=gu.DEV)
        nbytes = qg.qgemv_workspace_bytes(wtype, rows, cols, nvec)
        ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=gu.DEV) if nbytes else None
        cases.append((wtype, rows, cols, nvec, w, x, xq, xd, y, ws))

    def run():
        for wtype, rows, cols, nvec, w, x, xq, xd, y, ws in cases:
            qg.qgemv_quantize_act(x, xq, xd, cols, nvec)
            qg.qgemv_batch(wtype, w, xq, xd, y, rows, cols, nvec, workspace=ws)

    def set_inputs(seed):
        r = np.random.default_rng(seed)
        xs = []
        for c in cases:
            xv = (r.standard_normal(tuple(c[5].shape)) * 2.0).astype(np.float32)
            c[5].copy_(torch.from_numpy(xv).to(gu.DEV))
            xs.append(xv)
        return xs

    def outputs():
        return [gu.host(c[8]).copy() for c in cases]

    def clear():
        for c in cases:
            c[8].fill_(float("nan"))

    set_inputs(0)
    run()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        qg.qgemv_graph_begin()
        run()
        graph = qg.qgemv_graph_end()
    torch.cuda.synchronize()
    kernels, others = graph.nodes()
    assert others == 0 and kernels >= 2 * len(cases)
    for rep in range(1, 4):
        _say("matrix-core routes, replay", rep)
        xs = set_inputs(rep)
        clear()
        graph.launch()
        torch.cuda.synchronize()
        replayed = outputs()
        clear()
        run()
        torch.cuda.synchronize()
        _same_bits(replayed, outputs())
    # the last replay's outputs against the oracle, on the first and last 128 rows
    for (wtype, rows, cols, nvec, w, *_), xv, yv in zip(cases, xs, replayed):
        wbuf = gu.host(w)
        rq, rd = oracle.quantize_act(xv)
        for lo, hi in ((0, 128), (rows - 128, rows)):
            ref = oracle.gemv(wtype, oracle.row_slice(wtype, wbuf, rows, cols, lo, hi), hi - lo,
                              cols, rq, rd)
            gu.assert_within_bound(yv[:, lo:hi], ref)
    graph.close()


def test_graph_capture_errors():
    import torch
    import block_quantized_weight_act_amd as qg
    side = torch.cuda.Stream()
    with pytest.raises(qg.QgemvError):
        qg.qgemv_graph_begin(0)                  # the null stream cannot capture
    with pytest.raises(qg.QgemvError):
        qg.qgemv_graph_end(side)                 # not capturing

    cols, rows = 512, 40
    rng = np.random.default_rng(11)
    buf = oracle.quantize_q4k((rng.standard_normal((rows, cols)) * 0.02).astype(np.float32))
    w = gu.dev(buf)
    x_host = rng.standard_normal((1, cols)).astype(np.float32)
    x = gu.dev(x_host)
    y = torch.zeros((1, rows), dtype=torch.float32, device=gu.DEV)
    torch.cuda.synchronize()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        qg.qgemv_graph_begin()
        with pytest.raises(qg.QgemvError):
            qg.qgemv_graph_begin()              # already capturing
        with pytest.raises(qg.QgemvError):      # failed argument checks record nothing
            qg.qgemv_fused("q4k", w, x, y, rows, cols + 32, 1)
        qg.qgemv_fused("q4k", w, x, y, rows, cols, 1)
        graph = qg.qgemv_graph_end()
    torch.cuda.synchronize()
    assert graph.nodes() == (1, 0)
    for _ in range(3):
        y.fill_(float("nan"))
        graph.launch()
        torch.cuda.synchronize()
        rq, rd = oracle.quantize_act(x_host)
        gu.assert_within_bound(gu.host(y), oracle.gemv("q4k", buf, rows, cols, rq, rd))
    graph.close()
    graph.close()                               # a second close is a no-op
