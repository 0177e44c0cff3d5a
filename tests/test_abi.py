"""The C-ABI library's argument checks on the CPU: bad arguments are rejected on the host
before anything reaches the GPU. The calls pass fake device addresses, and no call here
passes validation, so nothing is ever launched. Because a future validation slip would turn
such a call into a launch at a wild address, the module does not run in a process that sees
a GPU (the exports and host-only helpers are checked in test_abi_exports.py)."""

import ctypes

import pytest
import torch

import block_quantized_weight_act_amd as qg

# device_count() does not initialise the GPU runtime
pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="fake device addresses are only passed where no GPU is visible")

EINVAL, EALIGN, EWORKSPACE = 1, 2, 3
A = 1 << 40          # a fake, 256-byte aligned "device address" (never dereferenced)


def test_status_strings_and_sizes():
    lib = qg._load()
    assert qg.qgemv_version() >= 100
    for s in range(5):
        assert lib.qgemv_status_string(s)
    assert qg.qgemv_weight_bytes("q4k", 3, 512) == 3 * 2 * 144
    assert qg.qgemv_weight_bytes("q6k", 3, 512) == 3 * 2 * 210
    assert qg.qgemv_weight_bytes("q4k", 3, 500) == 0
    assert qg.qgemv_workspace_bytes("q4k", 262144, 1536, 1) == 0


def _call_batch(wtype=1, w=A, xq=A + (1 << 30), xd=A + (2 << 30), y=A + (3 << 30), rows=64,
                cols=1024, nvec=1, ws=None, wsb=0):
    lib = qg._load()
    return lib.qgemv_batch(wtype, w, xq, xd, y, rows, cols, nvec, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(wtype=5), EINVAL), (dict(wtype=0), EINVAL), (dict(w=None), EINVAL), (dict(y=None), EINVAL),
    (dict(cols=1000), EINVAL), (dict(cols=0), EINVAL), (dict(rows=0), EINVAL),
    (dict(nvec=0), EINVAL), (dict(nvec=257), EINVAL), (dict(w=A + 8), EALIGN),
    (dict(xq=A + (1 << 30) + 4), EALIGN), (dict(y=A + (3 << 30) + 2), EALIGN),
    (dict(y=A + 64), EINVAL),              # output overlapping the weights
    (dict(rows=1 << 31), EINVAL),
])
def test_batch_rejects_bad_arguments(kw, status):
    assert _call_batch(**kw) == status


def _call_i8mc(w=A, xq=A + (1 << 30), xd=A + (2 << 30), y=A + (3 << 30), rows=64, cols=1024,
               nvec=4, ws=None, wsb=0):
    return qg._load().qgemv_batch_i8mc(w, xq, xd, y, rows, cols, nvec, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(w=None), EINVAL), (dict(y=None), EINVAL), (dict(cols=1000), EINVAL),
    (dict(cols=0), EINVAL), (dict(rows=0), EINVAL), (dict(nvec=0), EINVAL),
    (dict(nvec=17), EINVAL), (dict(w=A + 8), EALIGN), (dict(xq=A + (1 << 30) + 4), EALIGN),
    (dict(y=A + 64), EINVAL), (dict(rows=1 << 31), EINVAL),
    (dict(cols=4096), EWORKSPACE),                       # two column splits need partial sums
    (dict(cols=4096, ws=A + (4 << 30), wsb=2 * 4 * 64 * 4 - 4), EWORKSPACE),
    (dict(cols=4096, ws=A + (4 << 30) + 2, wsb=1 << 20), EALIGN),
    (dict(cols=4096, ws=A + (3 << 30), wsb=1 << 20), EINVAL),   # workspace over y
])
def test_i8mc_rejects_bad_arguments(kw, status):
    assert _call_i8mc(**kw) == status


def test_i8mc_workspace_and_routing():
    """Partial sums only past one split of 2048 columns; qgemv_batch takes this path (and its
    workspace) from 4 vectors on tensors of at least 32 MiB."""
    assert qg.qgemv_i8mc_workspace_bytes(64, 2048, 8) == 0
    assert qg.qgemv_i8mc_workspace_bytes(64, 4096, 3) == 2 * 3 * 64 * 4
    assert qg.qgemv_i8mc_workspace_bytes(10, 6144, 8) == 3 * 8 * 10 * 4
    assert qg.qgemv_i8mc_workspace_bytes(64, 2304, 2) == 2 * 2 * 64 * 4   # 9 super-blocks: 6 + 3
    assert qg.qgemv_i8mc_workspace_bytes(64, 4096, 17) == 0                # invalid
    assert qg.qgemv_i8mc_workspace_bytes(64, 4096, 16) == 2 * 16 * 64 * 4
    big = (65536, 4096)                                                    # 144 MiB of Q4_K
    assert qg.qgemv_workspace_bytes("q4k", *big, 4) == qg.qgemv_i8mc_workspace_bytes(*big, 4)
    # the routing thresholds: 16 MiB at 8 vectors (16384 x 2048: 18 MiB), 128 MiB at 3
    assert qg.qgemv_workspace_bytes("q4k", 16384, 4096, 8) == qg.qgemv_i8mc_workspace_bytes(16384, 4096, 8)
    assert qg.qgemv_workspace_bytes("q4k", 16384, 4096, 3) != qg.qgemv_i8mc_workspace_bytes(16384, 4096, 3)
    lib = qg._load()
    # no workspace: refused as the integer path refuses it, before any launch
    assert lib.qgemv_batch(1, A, A + (1 << 30), A + (2 << 30), A + (3 << 30), *big, 4, None, 0,
                           None) == EWORKSPACE
    fused = lib.qgemv_fused_i8mc
    assert fused(A, A + (1 << 30) + 4, None, None, A + (3 << 30), 64, 1024, 4, None, 0, None) == EALIGN
    assert fused(A, A + (1 << 30), A + (4 << 30), None, A + (3 << 30), 64, 1024, 4, None, 0,
                 None) == EINVAL                                           # one output of two
    assert lib.qgemv_debug_partials_i8mc(A, A + (1 << 30), A + (2 << 30), None, A + (4 << 30), 64,
                                         1024, 4, None) == EINVAL


def test_routes():
    assert qg.qgemv_route("q4k", 262144, 1536, 1) == "vector"
    assert qg.qgemv_route("q4k", 16384, 2048, 8) == "i8mc"
    assert qg.qgemv_route("q4k", 16384, 2048, 4) == "mc32"      # 4 vectors on 16-96 MiB
    assert qg.qgemv_route("q4k", 16384, 2048, 3) == "vector"
    assert qg.qgemv_route("q4k", 16384, 4096, 4) == "vector"    # two splits
    assert qg.qgemv_route("q4k", 8192, 2048, 4) == "vector"     # under 16 MiB
    assert qg.qgemv_route("q4k", 262144, 1536, 3) == "i8mc"
    assert qg.qgemv_route("q6k", 262144, 1536, 8) == "mc32"         # few Q6_K vectors
    assert qg.qgemv_route("q6k", 262144, 1536, 4) == "mc32"
    assert qg.qgemv_route("q6k", 262144, 1536, 3) == "vector"
    assert qg.qgemv_route("q6k", 65536, 2048, 8) == "mc32"
    assert qg.qgemv_route("q6k", 65536, 2048, 7) == "vector"
    assert qg.qgemv_route("q6k", 16384, 4096, 8) == "vector"
    assert qg.qgemv_route("q4k", 16384, 2048, 64) == "mc"
    assert qg.qgemv_route("q4k", 16384, 2048, 12) == "mc32"         # 9..12 on < 128 MiB: the
    assert qg.qgemv_route("q4k", 16384, 2048, 13) == "i8mc"         # few-vector kernel; else
    assert qg.qgemv_route("q4k", 262144, 1536, 12) == "i8mc"        # the Q4_K integer kernel
    assert qg.qgemv_route("q4k", 512, 512, 16) == "i8mc"
    assert qg.qgemv_route("q4k", 512, 512, 17) == "mc"
    assert qg.qgemv_route("q40", 16384, 2048, 64) == "mc32"
    assert qg.qgemv_route("q80", 262144, 1536, 9) == "mc32"
    assert qg.qgemv_route("q80", 262144, 1536, 8) == "mc32"         # few vectors: 8 on >= 256 Mi
    assert qg.qgemv_route("q80", 262144, 1536, 7) == "vector"
    assert qg.qgemv_route("q80", 65536, 2048, 8) == "vector"
    assert qg.qgemv_route("q40", 262144, 1536, 2) == "vector"       # Q4_0: from 4 on >= 32 Mi
    assert qg.qgemv_route("q40", 262144, 1536, 3) == "mc32"         # (3 on >= 256 Mi)
    assert qg.qgemv_route("q40", 65536, 2048, 3) == "vector"
    assert qg.qgemv_route("q40", 262144, 1536, 4) == "mc32"
    assert qg.qgemv_route("q40", 16384, 2048, 4) == "mc32"
    assert qg.qgemv_route("q40", 16000, 2048, 8) == "vector"
    assert qg.qgemv_route("q40", 16384, 4096, 7) == "vector"        # two splits: from 8
    assert qg.qgemv_route("q40", 16384, 4096, 8) == "mc32"
    assert qg.qgemv_route("q6k", 16384, 2048, 64) == "mc32"
    # Q8_0, Q4_0, Q6_K: the matrix cores from 32 vectors, from 16 on >= 24 Mi weights, from 9
    # on >= 48 Mi weights; groups of 8 on the vector kernel below
    assert qg.qgemv_route("q80", 2048, 8192, 9) == "mc32"           # 9..16: from 16 Mi weights
    assert qg.qgemv_route("q80", 2048, 4096, 9) == "grouped"
    assert qg.qgemv_route("q80", 2048, 8192, 24) == "grouped"
    assert qg.qgemv_route("q80", 2048, 8192, 32) == "mc32"
    assert qg.qgemv_route("q6k", 16384, 2048, 9) == "mc32"
    assert qg.qgemv_route("q80", 65536, 2048, 12) == "mc32"         # (the 32 x 32 x 32 kernel)
    assert qg.qgemv_route("q6k", 16384, 2048, 16) == "mc32"
    assert qg.qgemv_route("q40", 65536, 1536, 9) == "mc32"
    assert qg.qgemv_route("q40", 16384, 1536, 15) == "mc32"
    assert qg.qgemv_route("q40", 4096, 1536, 15) == "grouped"
    assert qg._load().qgemv_route(1, 8, 500, 1) == 0
    assert qg._load().qgemv_route(1, 8, 512, 300) == 0


def test_mc32_tile_names_the_kernel():
    """Which kernel qgemv_batch_mc32 runs: the 16 x 16 x 64 one for 1..8 vectors, for Q4_K, and
    for 9..16 where the route rule gives it; the 32 x 32 x 32 ones above 16 vectors and on
    small tensors; none where the entry point does not take the shape."""
    assert qg.qgemv_mc32_tile("q40", 65536, 2048, 8) == 16
    assert qg.qgemv_mc32_tile("q40", 65536, 2048, 16) == 16
    assert qg.qgemv_mc32_tile("q40", 65536, 2048, 17) == 32
    assert qg.qgemv_mc32_tile("q40", 1024, 1024, 12) == 32        # under 16 Mi weights
    assert qg.qgemv_mc32_tile("q80", 65536, 2048, 12) == 32       # Q8_0 9..15 on 48..256 Mi
    assert qg.qgemv_mc32_tile("q80", 65536, 2048, 16) == 16
    assert qg.qgemv_mc32_tile("q4k", 65536, 2048, 12) == 16
    assert qg.qgemv_mc32_tile("q4k", 65536, 2048, 17) == 0
    assert qg.qgemv_mc32_tile("q6k", 1024, 1000, 4) == 0          # not whole super-blocks


def test_grouped_workspace_covers_the_last_group():
    """Groups of 8 vectors share one workspace: it must hold the last, smaller group's partial
    sums too when that group's plan splits the columns and the full groups' does not."""
    rows, cols = 300, 1056
    assert qg.qgemv_route("q80", rows, cols, 9) == "grouped"
    p8, p1 = qg.qgemv_plan_for("q80", rows, cols, 8), qg.qgemv_plan_for("q80", rows, cols, 1)
    need1 = qg.qgemv_plan_workspace_bytes(p1, rows, cols, 1)
    need8 = qg.qgemv_plan_workspace_bytes(p8, rows, cols, 8)
    assert need1 > 0
    assert qg.qgemv_workspace_bytes("q80", rows, cols, 9) == max(need1, need8)
    for nvec in (9, 12, 17, 24, 33):
        rest = nvec % 8
        want = qg.qgemv_plan_workspace_bytes(qg.qgemv_plan_for("q40", 16384, 1536, 8), 16384, 1536, 8)
        if rest:
            want = max(want, qg.qgemv_plan_workspace_bytes(
                qg.qgemv_plan_for("q40", 16384, 1536, rest), 16384, 1536, rest))
        if qg.qgemv_route("q40", 16384, 1536, nvec) == "grouped":
            assert qg.qgemv_workspace_bytes("q40", 16384, 1536, nvec) == want


def test_split_plan_without_workspace_is_rejected():
    lib = qg._load()
    plan = qg.Plan(16, 1, 4, 4, 0)
    rows, cols = 64, 4096
    assert lib.qgemv_plan_workspace_bytes(ctypes.byref(plan), rows, cols, 1) == 8 * rows * 4
    st = lib.qgemv_batch_plan(1, A, A + (1 << 30), A + (2 << 30), A + (3 << 30), rows, cols, 1,
                              ctypes.byref(plan), None, 0, None)
    assert st == EWORKSPACE
    st = lib.qgemv_batch_plan(1, A, A + (1 << 30), A + (2 << 30), A + (3 << 30), rows, cols, 1,
                              ctypes.byref(plan), A + (4 << 30), 100, None)
    assert st == EWORKSPACE
    bad = qg.Plan(12, 1, 4, 4, 0)
    assert lib.qgemv_batch_plan(1, A, A + (1 << 30), A + (2 << 30), A + (3 << 30), rows, cols, 1,
                                ctypes.byref(bad), None, 0, None) == EINVAL
    for wide in (qg.Plan(16, 1, 8, 4, 0),              # a narrow slice: at most 4 waves
                 qg.Plan(64, 3, 9, 4, 0), qg.Plan(64, 3, 0, 4, 0)):
        assert lib.qgemv_batch_plan(1, A, A + (1 << 30), A + (2 << 30), A + (3 << 30), rows,
                                    cols, 1, ctypes.byref(wide), None, 0, None) == EINVAL
    toomany = qg.Plan(16, 4, 4, 4, 0)                  # 3 vectors x 4 chunks: not compiled
    assert lib.qgemv_batch_plan(1, A, A + (1 << 30), A + (2 << 30), A + (3 << 30), rows, cols, 3,
                                ctypes.byref(toomany), None, 0, None) == EINVAL


def test_other_entry_points_reject_bad_arguments():
    lib = qg._load()
    assert lib.qgemv_quantize_act(A, A + (1 << 30), A + (2 << 30), 48, 1, None) == EINVAL
    assert lib.qgemv_quantize_act(A + 4, A + (1 << 30), A + (2 << 30), 64, 1, None) == EALIGN
    assert lib.qgemv_quantize_act(None, A, A, 64, 1, None) == EINVAL
    assert lib.qgemv_q4k(A, A + (1 << 30), A + (2 << 30), None, 8, 256, None, 0, None) == EINVAL
    assert lib.qgemv_q6k(A + 2, A + (1 << 30), A + (2 << 30), A + (3 << 30), 8, 256, None, 0,
                         None) == EALIGN
    assert lib.qgemv_debug_partials(1, A, A + (1 << 30), A + (2 << 30), None, A, 8, 256, 1,
                                    None, 0, None) == EINVAL
    # the float matrix-core debug form (17+ vectors) needs the workspace
    assert lib.qgemv_debug_partials(1, A, A + (1 << 30), A + (2 << 30), A + (3 << 30),
                                    A + (4 << 30), 8, 256, 17, None, 0, None) == EWORKSPACE
    assert lib.qgemv_quantize_weights(2, A, A + 64, 8, 256, None) == EINVAL   # overlap
    assert lib.qgemv_quantize_weights(2, A + 4, A + (1 << 30), 8, 256, None) == EALIGN
    assert lib.qgemv_quantize_weights(5, A, A + (1 << 30), 8, 256, None) == EINVAL
    W = A + (1 << 30)
    rows = lib.qgemv_quantize_weights_rows
    assert rows(1, A, W, 8, 256, 0, 0, None) == EINVAL        # empty range
    assert rows(1, A, W, 8, 256, -1, 2, None) == EINVAL       # starts before row 0
    assert rows(1, A, W, 8, 256, 7, 2, None) == EINVAL        # ends past the last row
    assert rows(1, A, W, 8, 256, 1 << 40, 2, None) == EINVAL
    assert rows(2, A + 4, W, 8, 256, 0, 8, None) == EALIGN
    assert rows(2, A, A + 64, 8, 256, 4, 4, None) == EINVAL   # tensor over the rows


def test_fused_launch_count():
    """The one-launch kernel unless code outputs are wanted and the slice each workgroup
    quantizes (the whole row where the column split runs inside the workgroup) is more than
    32 elements per lane, or the workgroups together repeat its quantization for over 16K
    elements per CU with the slice over a tenth of a workgroup's weight bytes (then quantize
    once, then the product), and always on the integer matrix-core path (Q4_K, several
    vectors, a large tensor)."""
    assert qg.qgemv_fused_launches("q4k", 262144, 1536, 1) == 1      # 25K per CU, slice 0.03
    assert qg.qgemv_fused_launches("q4k", 8192, 2048, 1) == 1
    assert qg.qgemv_fused_launches("q6k", 2048, 8192, 1) == 1       # 8192 columns, 8 waves: 16
    assert qg.qgemv_fused_launches("q4k", 1536, 6144, 1) == 1       # 6144 columns, 8 waves: 12
    assert qg.qgemv_fused_launches("q6k", 2048, 8192, 2) == 1       # two vectors: 32, 16K
    assert qg.qgemv_fused_launches("q4k", 8192, 2048, 8) == 1       # 8 vectors, 8 waves: 32, 16K
    assert qg.qgemv_fused_launches("q4k", 8192, 2048, 4) == 1       # 4 vectors, 8 waves: 16
    assert qg.qgemv_fused_launches("q4k", 2048, 8192, 3) == 2       # split in two: the row, 48
    assert qg.qgemv_fused_launches("q4k", 1536, 6144, 4) == 2       # split in three: the row, 64
    assert qg.qgemv_fused_launches("q4k", 16384, 4096, 2) == 2      # 16 per lane, 33K per CU
    assert qg.qgemv_fused_launches("q4k", 4096, 16384, 1) == 2      # 512 workgroups x 16384
    assert qg.qgemv_fused_launches("q4k", 16384, 2048, 8) == 2
    assert qg.qgemv_fused_launches("q4k", 262144, 1536, 8) == 2      # integer matrix cores
    assert qg.qgemv_fused_launches("q4k", 262144, 1536, 8, with_outputs=False) == 1
    assert qg.qgemv_fused_launches("q4k", 16384, 2048, 8, with_outputs=False) == 1
    assert qg._load().qgemv_fused_launches(1, 0, 256, 1, 1) == 0
    assert qg._load().qgemv_fused_launches(5, 8, 256, 1, 1) == 0


def test_fused_rejects_bad_arguments():
    lib = qg._load()
    X, Q, D, Y = A + (1 << 30), A + (2 << 30), A + (5 << 30), A + (3 << 30)
    assert lib.qgemv_fused(1, A, None, None, None, Y, 8, 256, 1, None, 0, None) == EINVAL
    assert lib.qgemv_fused(1, A, X + 4, None, None, Y, 8, 256, 1, None, 0, None) == EALIGN
    assert lib.qgemv_fused(1, A, X, Q, None, Y, 8, 256, 1, None, 0, None) == EINVAL   # half the outputs
    assert lib.qgemv_fused(1, A, X, Q + 2, D, Y, 8, 256, 1, None, 0, None) == EALIGN
    assert lib.qgemv_fused(1, A, X, Q, D, X + 64, 8, 256, 1, None, 0, None) == EINVAL  # y over x
    assert lib.qgemv_fused(1, A, X, X + 16, D, Y, 8, 256, 1, None, 0, None) == EINVAL  # codes over x
    assert lib.qgemv_fused(5, A, X, None, None, Y, 8, 256, 1, None, 0, None) == EINVAL


def _mats(*specs):
    """ctypes array from (wtype, rows, w, y, reserved) tuples."""
    arr = (qg.Matrix * max(1, len(specs)))()
    for i, (t, rows, w, y, *rest) in enumerate(specs):
        arr[i] = qg.Matrix(t, rest[0] if rest else 0, rows, w, y)
    return arr


def test_multi_rejects_bad_arguments():
    lib = qg._load()
    XQ, XD = A + (1 << 30), A + (2 << 30)
    W1, W2, Y1, Y2 = A + (3 << 30), A + (4 << 30), A + (5 << 30), A + (6 << 30)
    good = [(1, 64, W1, Y1), (2, 32, W2, Y2)]

    def call(specs, n=None, cols=1536, nvec=1, xq=XQ, xd=XD):
        return lib.qgemv_multi(_mats(*specs), len(specs) if n is None else n, xq, xd, cols, nvec,
                               None)

    assert call(good, n=0) == EINVAL
    assert call(good * 5, n=9) == EINVAL                            # more than 8 matrices
    assert lib.qgemv_multi(None, 1, XQ, XD, 1536, 1, None) == EINVAL
    assert call([(5, 64, W1, Y1)]) == EINVAL                        # weight type
    assert call([(1, 64, W1, Y1, 1)]) == EINVAL                     # reserved field set
    assert call([(1, 0, W1, Y1)]) == EINVAL                         # no rows
    assert call([(1, 64, None, Y1)]) == EINVAL
    assert call([(1, 64, W1, None)]) == EINVAL
    assert call(good, cols=1000) == EINVAL
    # a row wider than one pass is split into at most a workgroup's waves (8) of chunks
    assert call(good, cols=65536 + 256) == EINVAL                   # 1 vector: 8 x 256 chunks
    assert call(good, cols=32768 + 256, nvec=3) == EINVAL           # 3-4 vectors: 8 x 128
    assert call(good, cols=16384 + 256, nvec=5) == EINVAL           # 5-8 vectors: 8 x 64
    assert call(good, xq=None) == EINVAL
    assert call(good, xq=XQ + 4) == EALIGN
    assert call([(1, 64, W1 + 8, Y1)]) == EALIGN
    assert call([(1, 64, W1, Y1 + 2)]) == EALIGN
    assert call([(1, 64, W1, W1 + 64)]) == EINVAL                   # y over the weights
    assert call([(1, 64, W1, Y1), (2, 32, W2, W1 + 256)]) == EINVAL # y over another's weights
    assert call([(1, 64, W1, Y1), (2, 32, W2, Y1 + 64)]) == EINVAL  # two outputs overlap
    assert call([(1, 64, W1, XQ + 64)]) == EINVAL                   # y over the codes
    # the fused form
    X, Q, D = A + (7 << 30), A + (8 << 30), A + (9 << 30)
    f = lib.qgemv_multi_fused
    assert f(_mats(*good), 2, None, None, None, 1536, 1, None) == EINVAL
    assert f(_mats(*good), 2, X + 4, None, None, 1536, 1, None) == EALIGN
    assert f(_mats(*good), 2, X, Q, None, 1536, 1, None) == EINVAL      # half the outputs
    assert f(_mats(*good), 2, X, Q + 2, D, 1536, 1, None) == EALIGN
    assert f(_mats(*good), 2, X, X + 16, D, 1536, 1, None) == EINVAL    # codes over x
    assert f(_mats(*good), 2, X, W1 + 16, D, 1536, 1, None) == EINVAL   # codes over weights
    assert f(_mats((1, 64, W1, X + 64)), 1, X, None, None, 1536, 1, None) == EINVAL  # y over x
    # 65536 columns, 8 chunks: their slices (73728 bytes) exceed the LDS limit, so the fused
    # form needs code outputs to quantize into (16-byte aligned ones)
    assert f(_mats(*good), 2, X, None, None, 65536, 1, None) == EINVAL
    assert f(_mats(*good), 2, X, Q + 4, D, 65536, 1, None) == EINVAL


def test_multi_geometry():
    """One pass over the row, fewest idle lanes, more chunks per lane preferred (at most 3 with
    2 vectors); a wider row takes the one-matrix planner's geometry (each further pass priced
    as 2% idle lanes, 15% from 5 vectors), its chunks split inside the workgroup."""
    assert qg.qgemv_multi_geometry(1536, 1) == (16, 3)
    assert qg.qgemv_multi_geometry(8192, 1) == (64, 4)
    assert qg.qgemv_multi_geometry(2048, 8) == (64, 1)
    assert qg.qgemv_multi_geometry(256, 1) == (8, 1)
    assert qg.qgemv_multi_geometry(4096, 3) == (64, 2)
    assert qg.qgemv_multi_geometry(8448, 1) == (32, 3)      # 264 chunks: 3 passes of 96
    assert qg.qgemv_multi_geometry(16384, 1) == (64, 4)     # 2 passes
    assert qg.qgemv_multi_geometry(4096, 5) == (64, 1)      # 2 passes
    assert qg.qgemv_multi_geometry(16384, 8) == (64, 1)     # 8 passes: 8 waves
    assert qg.qgemv_multi_geometry(14336, 1) == (64, 4)     # not 7 passes of 16 x 4: 4 waves
    assert qg.qgemv_multi_geometry(14336, 2) == (32, 2)     # 7 passes, 8 waves (2 vectors:
    assert qg.qgemv_multi_geometry(2048, 2) == (32, 2)      # at most 3 chunks per lane)
    assert qg.qgemv_multi_geometry(2048, 1) == (16, 4)
    lib = qg._load()
    t, nc = ctypes.c_int32(), ctypes.c_int32()
    assert lib.qgemv_multi_geometry(65536 + 256, 1, ctypes.byref(t), ctypes.byref(nc)) == EINVAL
    assert lib.qgemv_multi_geometry(16384 + 256, 5, ctypes.byref(t), ctypes.byref(nc)) == EINVAL
    assert lib.qgemv_multi_geometry(1536, 1, None, ctypes.byref(nc)) == EINVAL


def test_graph_entry_points_reject_bad_arguments_on_the_host():
    """Null graph or stream arguments are refused before any HIP call."""
    lib = qg._load()
    h = ctypes.c_void_p(123)
    assert lib.qgemv_graph_begin(None) == EINVAL                     # the null stream
    assert lib.qgemv_graph_end(None, ctypes.byref(h)) == EINVAL
    assert h.value is None                                           # cleared on error
    assert lib.qgemv_graph_end(A, None) == EINVAL
    assert lib.qgemv_graph_launch(None, None) == EINVAL
    k, o = ctypes.c_int64(), ctypes.c_int64()
    assert lib.qgemv_graph_nodes(None, ctypes.byref(k), ctypes.byref(o)) == EINVAL
    assert lib.qgemv_graph_destroy(None) == 0


def test_matrix_core_path_limits_on_the_host():
    """More than 8 vectors: Q4_K only, at most QGEMV_MAX_BATCH, workspace sized for its split;
    all refused before any launch."""
    lib = qg._load()
    assert qg.qgemv_workspace_bytes("q4k", 256, 2048, 64) > 0          # few rows: split
    # enough rows: no split, only the staged activation tiles (8 super-blocks x 64 vectors)
    assert qg.qgemv_workspace_bytes("q4k", 1 << 16, 2048, 64) == 8 * 2 * 18432
    # Q6_K takes the plan of the 32-weight formats' matrix-core path: 2 row tiles of 128 rows,
    # 8 splits of one 8-block step
    assert qg.qgemv_workspace_bytes("q6k", 256, 2048, 64) == 8 * 64 * 256 * 4
    assert qg.qgemv_workspace_bytes("q6k", 256, 2048, 64) == qg.qgemv_workspace_bytes("q80", 256, 2048, 64)
    assert qg.qgemv_workspace_bytes("q4k", 256, 2048, 257) == 0
    assert _call_batch(nvec=257) == EINVAL
    assert _call_batch(wtype=2, nvec=257) == EINVAL
    assert _call_batch(wtype=3, nvec=9, y=None) == EINVAL
    assert _call_batch(wtype=4, nvec=40, xq=A + (1 << 30) + 4) == EALIGN
    assert _call_batch(nvec=64, rows=256, cols=2048) == EWORKSPACE
    assert _call_batch(nvec=64, xq=A + (1 << 30) + 4) == EALIGN
    plan = qg.Plan()
    assert lib.qgemv_plan_for(1, 64, 1024, 9, ctypes.byref(plan)) == EINVAL


def test_mc32_workspace_and_limits():
    """Q8_0 / Q4_0 with many vectors: partial sums only when the columns are split (few rows),
    refused before any launch without them; more than 256 vectors refused."""
    assert qg.qgemv_workspace_bytes("q80", 262144, 1536, 64) == 0
    # 128-row workgroups (64 vectors): 128 row tiles, so the columns are split in 4
    assert qg.qgemv_workspace_bytes("q40", 16384, 2048, 64) == 4 * 64 * 16384 * 4
    assert _call_batch(wtype=3, rows=16384, cols=2048, nvec=64) == EWORKSPACE
    assert _call_batch(wtype=4, nvec=257) == EINVAL
    assert _call_batch(wtype=4, cols=1000, nvec=20) == EINVAL
    lib = qg._load()
    assert lib.qgemv_debug_partials(4, A, A + (1 << 30), A + (2 << 30), A + (3 << 30), None, 64,
                                    1024, 20, None, 0, None) == EINVAL          # no S
    for nvec in (4, 20):
        assert lib.qgemv_debug_partials_mc32(4, A, A + (1 << 30), A + (2 << 30), A + (3 << 30),
                                             None, 64, 1024, nvec, None) == EINVAL
    # the explicit entry point takes any shape of its formats with 9..256 vectors, and of Q8_0
    # and Q4_0 with 1..8 (splits of up to 64 blocks of 32 columns)
    X, D, Y = A + (1 << 30), A + (2 << 30), A + (3 << 30)
    mc = lib.qgemv_batch_mc32
    assert qg.qgemv_mc32_workspace_bytes("q80", 2048, 8192, 9) == 4 * 9 * 2048 * 4   # 16-vector kernel
    assert qg.qgemv_mc32_workspace_bytes("q80", 2048, 4096, 9) == 16 * 9 * 2048 * 4  # 32 x 32 x 32
    assert qg.qgemv_mc32_workspace_bytes("q80", 2048, 8192, 8) == 4 * 8 * 2048 * 4
    assert qg.qgemv_mc32_workspace_bytes("q40", 2048, 2048, 8) == 0
    assert qg.qgemv_mc32_workspace_bytes("q40", 2048, 8224, 3) == 5 * 3 * 2048 * 4
    assert qg.qgemv_mc32_workspace_bytes("q6k", 2048, 8192, 8) == 4 * 8 * 2048 * 4
    assert qg.qgemv_mc32_workspace_bytes("q4k", 2048, 8192, 64) == 0
    assert mc(2, A, X, D, Y, 2048, 8192, 8, None, 0, None) == EWORKSPACE     # Q6_K: its split
    assert mc(2, A, X, D, Y, 2048, 8192 + 32, 8, None, 0, None) == EINVAL    # Q6_K: whole 256s
    assert mc(4, A, X, D, Y, 2048, 8192, 8, None, 0, None) == EWORKSPACE     # its split
    assert mc(3, A, X, D, Y, 2048, 8192, 0, None, 0, None) == EINVAL
    assert mc(1, A, X, D, Y, 2048, 8192, 64, None, 0, None) == EINVAL        # Q4_K
    assert mc(2, A, X, D, Y, 2048, 1024 + 32, 64, None, 0, None) == EINVAL   # Q6_K: whole 256s
    assert mc(4, A, X, D, Y, 2048, 8192, 9, None, 0, None) == EWORKSPACE     # its split
    assert mc(4, A, X + 4, D, Y, 2048, 8192, 9, None, 0, None) == EALIGN


def test_scratch_entry_point_rejects_bad_arguments():
    """qgemv_batch_scratch refuses a bad type or shape, null pointers and shapes whose
    workspace exceeds the static scratch before it looks up anything."""
    lib = qg._load()
    X, Y = A + (1 << 30), A + (3 << 30)
    sc = lib.qgemv_batch_scratch
    assert sc(5, A, X, A + (2 << 30), Y, 64, 1024, 1, None) == EINVAL
    assert sc(1, A, X, A + (2 << 30), Y, 64, 1000, 1, None) == EINVAL
    assert sc(1, None, X, A + (2 << 30), Y, 64, 1024, 1, None) == EINVAL
    assert sc(1, A, X, A + (2 << 30), None, 64, 1024, 1, None) == EINVAL
    # 128 rows x 65536 columns x 256 vectors on the float matrix cores: 256 column splits of
    # partial sums (32 MiB) plus the staged tiles, beyond the 32 MiB scratch
    assert qg.qgemv_workspace_bytes("q4k", 128, 65536, 256) > qg.SCRATCH_BYTES
    assert sc(1, A, X, A + (2 << 30), Y, 128, 65536, 256, None) == EWORKSPACE


def test_fused_plan_rejects_bad_arguments():
    """qgemv_fused_plan refuses what qgemv_fused and qgemv_batch_plan refuse."""
    lib = qg._load()
    X, Y = A + (1 << 30), A + (3 << 30)
    fp = lib.qgemv_fused_plan
    plan = qg.Plan(64, 2, 4, 4, 0)
    assert fp(1, A, X, None, None, Y, 64, 8192, 1, None, None, 0, None) == EINVAL      # no plan
    assert fp(1, A, X, None, None, Y, 64, 8192, 1, ctypes.byref(plan), None, 0,
              None) == EWORKSPACE                                   # two column chunks
    assert fp(1, A, X + 4, None, None, Y, 64, 8192, 1, ctypes.byref(plan), None, 0,
              None) == EALIGN
    assert fp(1, A, X, A + (4 << 30), None, Y, 64, 8192, 1, ctypes.byref(plan), None, 0,
              None) == EINVAL                                       # one code output of two
    bad = qg.Plan(12, 1, 4, 4, 0)
    assert fp(1, A, X, None, None, Y, 64, 8192, 1, ctypes.byref(bad), None, 0, None) == EINVAL
