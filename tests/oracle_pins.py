"""Checks that pin the CPU oracle to facts that do not come from the oracle itself.

Each check takes a loaded oracle library (`lib`) so that the same checks can be
run against deliberately broken builds of the oracle (tests/test_oracle_mutants.py):
every planted mistake must make at least one of them fail.

What pins what:
  fp16 codec        numpy's IEEE binary16 conversions (a library routine), exhaustively.
  block layouts     hand-derived fixtures under tests/golden/ and single-field probes.
  activation codes  hand-worked blocks (ties to even, the scale as one division) and the
                    rounding bound |x - xd*q| <= xd/2.
  weight quantizers round-trip error bounds derived from the grid construction, and
                    nearest-code optimality of every stored code.
  integer GEMV      a float64 brute force over dequantized weights (every product is
                    exact), one-hot / constant / zero inputs (closed forms), and the
                    int32 extremes.
"""

from __future__ import annotations

import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ helpers --
def read_hex_fixture(name: str):
    params = {}
    data = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("params"):
                for item in line.split()[1:]:
                    k, v = item.split("=", 1)
                    params[k] = v
                continue
            data.extend(int(tok, 16) for tok in line.split())
    return params, np.array(data, dtype=np.uint8)


def read_probes():
    rows = []
    with open(os.path.join(GOLDEN, "layout_probes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fmt, byte, shift, width, field, value = line.split()
            name, idx = field[:-1].split("[")
            rows.append((fmt, int(byte), int(shift), int(width), name, int(idx), int(value)))
    return rows


def read_act_cases():
    cases = []
    with open(os.path.join(GOLDEN, "act_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            xs, qs, ds = (part.strip() for part in line.split("|"))
            x = np.zeros(32, np.float32)
            for tok in xs.split()[1:]:
                i, v = tok.split(":")
                x[int(i)] = np.float32(float(v))
            q = np.zeros(32, np.int8)
            for tok in qs.split()[1:]:
                i, v = tok.split(":")
                q[int(i)] = int(v)
            num, den = ds.split()[1].split("/")
            xd = np.float32(num) / np.float32(den)      # one IEEE float32 division (numpy)
            cases.append((x, q, xd))
    return cases


# --------------------------------------------------------------------- fp16 --
def check_fp16(lib):
    # half -> float, all 65536 codes, against numpy
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float32)
    got = oracle.f16_to_f32(h, lib=lib)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    # float -> half: every half value, every midpoint between neighbours (ties), a
    # little above and below each midpoint, and random float32 bit patterns
    finite = h[~nan & np.isfinite(ref)]
    vals = finite.view(np.float16).astype(np.float64)
    srt = np.unique(vals)
    mids = (srt[:-1] + srt[1:]) / 2.0
    mids32 = mids.astype(np.float32)
    rng = np.random.default_rng(7)
    rand = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    probe = np.concatenate([
        vals.astype(np.float32), mids32, np.nextafter(mids32, np.float32(np.inf)),
        np.nextafter(mids32, np.float32(-np.inf)), rand,
        np.array([65504.0, 65519.99, 65520.0, 65536.0, 2.0**-24, 2.0**-25, 2.0**-25 * 1.0001,
                  2.0**-26, 1e-30, -0.0, np.inf, -np.inf], dtype=np.float32)])
    probe = probe[~np.isnan(probe)]
    with np.errstate(over="ignore"):
        ref16 = probe.astype(np.float16).view(np.uint16)
    got16 = oracle.f32_to_f16(probe, lib=lib)
    bad = np.nonzero(ref16 != got16)[0]
    assert bad.size == 0, "fp16 mismatch at %r" % (probe[bad[:5]],)


# ------------------------------------------------------------------- layout --
def _q4k_params(p):
    sc = np.array([int(v) for v in p["sc"].split(",")], np.uint8)
    m = np.array([int(v) for v in p["m"].split(",")], np.uint8)
    i = np.arange(256)
    q = (i % 16) if p["q"] == "i%16" else (15 - i % 16)
    return int(p["d16"], 16), int(p["dmin16"], 16), sc, m, q.astype(np.uint8)


def check_layout_goldens(lib):
    for name in ("q4k_block_a.txt", "q4k_block_b.txt"):
        p, blk = read_hex_fixture(name)
        assert blk.size == 144
        d16, m16, sc, m, q = _q4k_params(p)
        # pack: the oracle's packer must produce the hand-derived bytes
        assert np.array_equal(oracle.q4k_pack_block(d16, m16, sc, m, q, lib=lib), blk), name
        # unpack: the oracle's reader must recover the parameters
        gd, gm, gsc, gmm, gq = oracle.q4k_unpack_block(blk, lib=lib)
        assert (gd, gm) == (d16, m16) and np.array_equal(gsc, sc) and np.array_equal(gmm, m)
        assert np.array_equal(gq, q), name
        # dequantize: closed form d * sc_j * q_i - dmin * m_j
        d = float(np.array([d16], np.uint16).view(np.float16)[0])
        dmin = float(np.array([m16], np.uint16).view(np.float16)[0])
        j = np.arange(256) // 32
        want = d * sc[j].astype(np.float64) * q - dmin * m[j].astype(np.float64)
        got = oracle.dequantize("q4k", oracle.q4k_tensor([blk], lib=lib), 1, 256, lib=lib)[0]
        assert np.array_equal(got, want), name

    p, body = read_hex_fixture("q6k_block_a.txt")
    assert body.size == 208
    i = np.arange(256)
    q = (i % 64).astype(np.uint8)
    sc = np.array([3 * (j - 8) for j in range(16)], np.int8)
    assert np.array_equal(oracle.q6k_pack_block(sc, q, lib=lib), body)
    gsc, gq = oracle.q6k_unpack_block(body, lib=lib)
    assert np.array_equal(gsc, sc) and np.array_equal(gq, q)
    d16 = int(p["d16"], 16)
    tensor = oracle.q6k_tensor([body], [d16], lib=lib)
    want = 0.25 * sc[i // 16].astype(np.float64) * (q.astype(np.float64) - 32)
    assert np.array_equal(oracle.dequantize("q6k", tensor, 1, 256, lib=lib)[0], want)


def check_qk_tensor_goldens(lib):
    """Q4_K and Q6_K planar tensors of two blocks, against hand-derived bytes.

    The writer (block images -> tensor) must produce the fixture's bytes, the reader
    (tensor -> block image) must recover each block from them, and the dequantizer must
    read the fixture tensor, as one row of two blocks and as two rows of one block, into
    the closed-form weights. This pins the order and offsets of every plane.
    """
    pt, data = read_hex_fixture("qk_tensors.txt")
    n4 = int(pt["q4k_bytes"])
    want4, want6 = data[:n4], data[n4:]
    assert want4.size == 2 * 144 and want6.size == 2 * 210
    i = np.arange(256)
    j32 = i // 32

    # Q4_K: block 0 = fixture A, block 1 as stated in the fixture's header comment
    _, img0 = read_hex_fixture("q4k_block_a.txt")
    img1 = np.array([0x00, 0x40, 0x00, 0x34, 0x11, 0x11, 0x11, 0x11, 0x22, 0x22, 0x22, 0x22,
                     0xAA, 0xAA, 0x00, 0x00] + [0xC3] * 128, np.uint8)
    q1 = np.where(i % 32 < 16, 3, 12).astype(np.uint8)
    assert np.array_equal(
        oracle.q4k_pack_block(0x4000, 0x3400, np.full(8, 33, np.uint8), np.full(8, 2, np.uint8),
                              q1, lib=lib), img1)
    t4 = oracle.q4k_tensor([img0, img1], lib=lib)
    assert np.array_equal(t4, want4)
    assert np.array_equal(oracle.q4k_get_block(want4, 2, 0, lib=lib), img0)
    assert np.array_equal(oracle.q4k_get_block(want4, 2, 1, lib=lib), img1)
    p0 = read_hex_fixture("q4k_block_a.txt")[0]
    _, _, sc0, m0, qa = _q4k_params(p0)
    w0 = 1.0 * sc0[j32].astype(np.float64) * qa - 0.5 * m0[j32].astype(np.float64)
    w1 = np.where(i % 32 < 16, 197.5, 791.5)
    got = oracle.dequantize("q4k", want4, 1, 512, lib=lib)[0]
    assert np.array_equal(got, np.concatenate([w0, w1]))
    got2 = oracle.dequantize("q4k", want4, 2, 256, lib=lib)
    assert np.array_equal(got2[0], w0) and np.array_equal(got2[1], w1)

    # Q6_K: block 0 = fixture A with d = 0.25, block 1 as stated in the fixture's comment
    _, body0 = read_hex_fixture("q6k_block_a.txt")
    sc1 = (np.arange(16) - 4).astype(np.int8)
    body1 = np.concatenate([np.full(128, 0xDD, np.uint8), np.full(64, 0xAA, np.uint8),
                            sc1.view(np.uint8)])
    assert np.array_equal(oracle.q6k_pack_block(sc1, np.full(256, 45, np.uint8), lib=lib), body1)
    t6 = oracle.q6k_tensor([body0, body1], [0x3400, 0x3800], lib=lib)
    assert np.array_equal(t6, want6)
    b0, d0 = oracle.q6k_get_block(want6, 2, 0, lib=lib)
    b1, d1 = oracle.q6k_get_block(want6, 2, 1, lib=lib)
    assert np.array_equal(b0, body0) and d0 == 0x3400
    assert np.array_equal(b1, body1) and d1 == 0x3800
    sc0 = np.array([3 * (j - 8) for j in range(16)], np.float64)
    v0 = 0.25 * sc0[i // 16] * ((i % 64) - 32.0)
    v1 = 6.5 * (i // 16 - 4.0)
    got = oracle.dequantize("q6k", want6, 1, 512, lib=lib)[0]
    assert np.array_equal(got, np.concatenate([v0, v1]))
    got2 = oracle.dequantize("q6k", want6, 2, 256, lib=lib)
    assert np.array_equal(got2[0], v0) and np.array_equal(got2[1], v1)


def check_layout_probes(lib):
    for fmt, byte, shift, width, name, idx, value in read_probes():
        size = {"q4k": 144, "q6k": 208, "q40": 18, "q80": 36}[fmt]
        blk = np.zeros(size, np.uint8)
        blk[byte] = ((1 << width) - 1) << shift
        if fmt == "q4k":
            _, _, sc, m, q = oracle.q4k_unpack_block(blk, lib=lib)
            fields = {"sc": sc.astype(int), "m": m.astype(int), "q": q.astype(int)}
        elif fmt == "q6k":
            sc, q = oracle.q6k_unpack_block(blk, lib=lib)
            fields = {"sc": sc.astype(int), "q": q.astype(int)}
        elif fmt == "q40":
            _, q = oracle.q40_unpack_block(blk, lib=lib)
            fields = {"q": q.astype(int)}
        else:
            _, q = oracle.q80_unpack_block(blk, lib=lib)
            fields = {"q": q.astype(int)}
        for fname, arr in fields.items():
            want = np.zeros_like(arr)
            if fname == name:
                want[idx] = value
            assert np.array_equal(arr, want), (fmt, byte, shift, fname)


def check_q32_layout_goldens(lib):
    """Q4_0 / Q8_0 block images and the planar two-block tensors, against hand-derived bytes."""
    t = np.arange(32)
    p, img = read_hex_fixture("q40_block_a.txt")
    assert img.size == 18
    q = np.where(t < 16, t, 31 - t).astype(np.uint8)
    assert np.array_equal(oracle.q40_pack_block(int(p["d16"], 16), q, lib=lib), img)
    d16, gq = oracle.q40_unpack_block(img, lib=lib)
    assert d16 == 0xB000 and np.array_equal(gq, q)
    p80, img80 = read_hex_fixture("q80_block_a.txt")
    assert img80.size == 36
    q8 = (4 * t - 64).astype(np.int8)
    assert np.array_equal(oracle.q80_pack_block(np.float32(0.5), q8, lib=lib), img80)
    d8, gq8 = oracle.q80_unpack_block(img80, lib=lib)
    assert d8 == np.float32(0.5) and np.array_equal(gq8, q8)
    # the planar tensors of two blocks each
    pt, data = read_hex_fixture("q32_tensors.txt")
    n40 = int(pt["q40_bytes"])
    want40, want80 = data[:n40], data[n40:]
    img1 = oracle.q40_pack_block(0x3C00, np.full(32, 8, np.uint8), lib=lib)
    t40 = oracle.q32_tensor("q40", [img, img1], lib=lib)
    assert np.array_equal(t40, want40)
    img81 = oracle.q80_pack_block(np.float32(2.0), np.ones(32, np.int8), lib=lib)
    t80 = oracle.q32_tensor("q80", [img80, img81], lib=lib)
    assert np.array_equal(t80, want80)
    assert np.array_equal(oracle.q32_get_block("q40", t40, 2, 1, lib=lib), img1)
    assert np.array_equal(oracle.q32_get_block("q80", t80, 2, 0, lib=lib), img80)
    # dequantization: the closed forms d * (q - 8) and d * q, block by block
    w40 = oracle.dequantize("q40", t40, 1, 64, lib=lib)[0]
    assert np.array_equal(w40[:32], -0.125 * (q.astype(np.float64) - 8))
    assert np.all(w40[32:] == 0.0)
    w80 = oracle.dequantize("q80", t80, 1, 64, lib=lib)[0]
    assert np.array_equal(w80[:32], 0.5 * q8.astype(np.float64))
    assert np.all(w80[32:] == 2.0)
    # the same tensors read as two rows of one block each
    assert np.array_equal(oracle.dequantize("q40", t40, 2, 32, lib=lib).reshape(-1), w40)


# -------------------------------------------------------------- activations --
def check_act_cases(lib):
    for x, q, xd in read_act_cases():
        gq, gd = oracle.quantize_act(x[None, :], lib=lib)
        assert np.array_equal(gq[0], q), (x, gq[0], q)
        assert gd[0, 0].view(np.uint32) == np.float32(xd).view(np.uint32)


def check_act_bounds(lib, seed=11):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((4, 4096)).astype(np.float32)
    x[0, :32] *= 1e-30                            # tiny but normal-range blocks
    x[1, 32:64] = 0.0                             # an all-zero block
    x[2] *= np.float32(1e6)
    xq, xd = oracle.quantize_act(x, lib=lib)
    assert xq.min() >= -127
    blocks = x.reshape(4, -1, 32).astype(np.float64)
    codes = xq.reshape(4, -1, 32).astype(np.float64)
    scale = xd.astype(np.float64)[:, :, None]
    # rounding bound: |x - xd*q| <= xd/2, up to the rounding of the two float32 operations
    err = np.abs(blocks - scale * codes)
    assert np.all(err <= scale * (0.5 + 1e-5))
    # the element of largest magnitude gets the code +-127
    amax_idx = np.abs(blocks).argmax(axis=2)
    top = np.take_along_axis(codes, amax_idx[:, :, None], axis=2)[:, :, 0]
    amax = np.abs(blocks).max(axis=2)
    assert np.all(np.abs(top[amax > 0]) == 127)
    assert np.all(xd[amax == 0] == 0) and np.all(codes[amax == 0] == 0)
    # scale = amax / 127 as one float32 division
    assert np.array_equal(xd, (amax.astype(np.float32) / np.float32(127.0)))
    # scaling the input by a power of two scales xd exactly and keeps the codes
    xq2, xd2 = oracle.quantize_act(x * np.float32(8.0), lib=lib)
    assert np.array_equal(xq2, xq) and np.array_equal(xd2, xd * np.float32(8.0))


def check_act_overflowing_inverse(lib):
    """127 / amax overflows float32 below amax = 127 / FLT_MAX (about 3.73e-37): such a block has
    no finite inverse, and its codes are all 0 (the amax = 0 rule) with xd = amax / 127. A block
    just above the threshold has a finite inverse and the usual codes (+-127 at its maximum). A
    zero element gets the code 0 in every block."""
    f32max = np.finfo(np.float32).max
    limit = np.float32(127.0) / np.float32(f32max)
    rng = np.random.default_rng(5)
    x = np.zeros((1, 32 * 6), np.float32)
    for b, amax in enumerate([1e-37, 3.7e-37, 3.8e-37, 1e-30, 1.5e-45, 2e-38]):
        blk = (rng.uniform(-1.0, 1.0, 32) * amax).astype(np.float32)
        blk[3] = np.float32(amax)
        blk[7] = 0.0
        x[0, 32 * b:32 * b + 32] = blk
    xq, xd = oracle.quantize_act(x, lib=lib)
    codes = xq.reshape(-1, 32)
    am = np.abs(x.reshape(-1, 32)).max(axis=1)
    assert np.array_equal(xd[0], am / np.float32(127.0))
    assert np.all(codes[:, 7] == 0)
    for b in range(6):
        with np.errstate(over="ignore", divide="ignore"):
            finite = np.isfinite(np.float32(127.0) / am[b])
        assert finite == (am[b] >= limit), b
        if finite:
            assert abs(int(codes[b, 3])) == 127, b
        else:
            assert not codes[b].any(), b
    # Q8_0 weights follow the same rule, block by block
    wq = oracle.q80_codes(oracle.quantize_q80(x, lib=lib), 1, x.shape[1]).reshape(-1, 32)
    assert np.array_equal(wq, codes)


# ------------------------------------------------------------- quantizers --
def _f16(h):
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float64)


def check_q4k_quantizer(lib, w):
    rows, cols = w.shape
    buf = oracle.quantize_q4k(w, lib=lib)
    nb = cols // 256
    blocks = oracle.blocks_of("q4k", buf, rows, cols, lib=lib)
    what = oracle.dequantize("q4k", buf, rows, cols, lib=lib).reshape(rows * nb, 8, 32)
    wb = w.astype(np.float64).reshape(rows * nb, 8, 32)
    d = _f16(blocks[:, 0:2].copy().view(np.uint16)[:, 0])
    dmin = _f16(blocks[:, 2:4].copy().view(np.uint16)[:, 0])
    sc = np.zeros((rows * nb, 8)); m = np.zeros((rows * nb, 8))
    for b in range(rows * nb):
        _, _, s_, m_, _ = oracle.q4k_unpack_block(blocks[b], lib=lib)
        sc[b], m[b] = s_, m_
    step = d[:, None] * sc
    off = dmin[:, None] * m
    # the sub-block's own range: s_j = (hi - lo) / 15 with lo = min(0, min w), o_j = -lo
    lo = np.minimum(0.0, wb.min(axis=2))
    s = (wb.max(axis=2) - lo) / 15
    o = -lo
    # sub-scales are the nearest multiples of the super-scales, unless clamped at 63
    assert np.all((np.abs(step - s) <= d[:, None] * (0.5 + 1e-6) + 1e-12 * s) | (sc == 63))
    assert np.all((np.abs(off - o) <= dmin[:, None] * (0.5 + 1e-6) + 1e-12 * o) | (m == 63))
    # round-trip bound from the grid construction: codes 0..15 span [-off, -off + 15 step];
    # a weight inside is within step/2, one above the top is within 15 (s - step) + |off - o|,
    # one below the bottom within |off - o| (without clamping: step/2 + 7.5 d + dmin/2)
    bound = step / 2 + 15 * np.maximum(0.0, s - step) + np.abs(off - o)
    slack = 1e-6 * (np.abs(wb).max(axis=2) + off + 15 * step)
    err = np.abs(wb - what).max(axis=2)
    assert np.all(err <= bound + slack), float((err - bound).max())
    # every code is a nearest grid point of its sub-block
    grid = step[:, :, None] * np.arange(16)[None, None, :] - (dmin[:, None] * m)[:, :, None]
    best = np.abs(wb[:, :, :, None] - grid[:, :, None, :]).min(axis=3)
    assert np.all(np.abs(wb - what) <= best + 1e-6 * (step[:, :, None] + 1e-30))
    # the super-scales make full use of the 6-bit range (normal fp16 super-scales)
    nz = d >= 2.0 ** -14
    assert np.all(sc.max(axis=1)[nz] >= 62)
    nzm = dmin >= 2.0 ** -14
    assert np.all(m.max(axis=1)[nzm] >= 62)
    return buf


def check_q6k_quantizer(lib, w, negate=False):
    rows, cols = w.shape
    if negate:
        # the negated-scale encoding must dequantize to exactly the same weights
        buf = oracle.quantize_q6k(w, negate_scales=True, lib=lib)
        ref = oracle.quantize_q6k(w, negate_scales=False, lib=lib)
        assert np.array_equal(oracle.dequantize("q6k", buf, rows, cols, lib=lib),
                              oracle.dequantize("q6k", ref, rows, cols, lib=lib))
        bodies, _ = oracle.blocks_of("q6k", buf, rows, cols, lib=lib)
        assert (bodies[:, 192:].view(np.int8) < 0).any()
        check_q6k_quantizer(lib, w, negate=False)
        return buf
    buf = oracle.quantize_q6k(w, negate_scales=False, lib=lib)
    nb = cols // 256
    bodies, dplane = oracle.blocks_of("q6k", buf, rows, cols, lib=lib)
    d = _f16(dplane)
    what = oracle.dequantize("q6k", buf, rows, cols, lib=lib).reshape(rows * nb, 16, 16)
    wb = w.astype(np.float64).reshape(rows * nb, 16, 16)
    sc = np.zeros((rows * nb, 16))
    for b in range(rows * nb):
        s_, _ = oracle.q6k_unpack_block(bodies[b], lib=lib)
        sc[b] = s_
    assert np.all(sc >= 0)
    step = d[:, None] * sc
    s = np.abs(wb).max(axis=2) / 31
    # sc_j is the nearest multiple of d to s_j = max|w| / 31, unless clamped at 127
    assert np.all((np.abs(step - s) <= d[:, None] * (0.5 + 1e-6) + 1e-12 * s) | (sc == 127))
    # round-trip bound: codes -32..31 span [-32 step, 31 step] and |w| <= 31 s, so a weight
    # is within step/2 of the grid or at most 31 (s - step) beyond it
    # (without clamping: step/2 + 15.5 d)
    bound = step / 2 + 31 * np.maximum(0.0, s - step)
    slack = 1e-6 * (np.abs(wb).max(axis=2) + 32 * step)
    err = np.abs(wb - what).max(axis=2)
    assert np.all(err <= bound + slack), float((err - bound).max())
    # every code is a nearest grid point of its sub-block
    grid = step[:, :, None] * (np.arange(64) - 32)[None, None, :]
    best = np.abs(wb[:, :, :, None] - grid[:, :, None, :]).min(axis=3)
    assert np.all(np.abs(wb - what) <= best + 1e-6 * (step[:, :, None] + 1e-30))
    # with a normal fp16 d (relative rounding <= 2^-11) the largest sub-scale reaches 126..127
    nz = d >= 2.0 ** -14
    assert np.all(sc.max(axis=1)[nz] >= 126)
    return buf


def check_q40_quantizer(lib, w):
    """Q4_0: the block's largest-magnitude weight sets d (it lands on code 0 up to the fp16
    rounding of d), every code is a nearest grid point d * (q - 8), and only weights beyond
    7.5 |d| on the opposite side are clipped (to code 15)."""
    rows, cols = w.shape
    buf = oracle.quantize_q40(w, lib=lib)
    n = rows * cols // 32
    imgs = np.stack([oracle.q32_get_block("q40", buf, n, i, lib=lib) for i in range(n)])
    d = _f16(imgs[:, :2].copy().view(np.uint16)[:, 0])
    wb = w.astype(np.float64).reshape(n, 32)
    what = oracle.dequantize("q40", buf, rows, cols, lib=lib).reshape(n, 32)
    codes = np.stack([oracle.q40_unpack_block(imgs[i], lib=lib)[1] for i in range(n)]).astype(int)
    # the scale: d * (0 - 8) reproduces the first largest-magnitude weight m
    idx = np.abs(wb).argmax(axis=1)
    m = wb[np.arange(n), idx]
    normal = np.abs(d) >= 2.0 ** -14
    assert np.all(np.abs(-8 * d - m)[normal] <= 8 * np.abs(d[normal]) * 2.0 ** -11)
    assert np.all(codes[np.arange(n), idx][normal] == 0)
    assert np.all(d[m == 0] == 0) and np.all(codes[m == 0] == 8)
    # nearest grid point among the 16 codes
    grid = d[:, None, None] * (np.arange(16) - 8)[None, None, :]
    best = np.abs(wb[:, :, None] - grid).min(axis=2)
    err = np.abs(wb - what)
    assert np.all(err <= best + 1e-6 * np.abs(d)[:, None] + 1e-300)
    # round-trip bound: |d|/2 inside the grid, and at most |w| - 7 |d| for clipped weights
    inside = np.abs(wb) <= 7.5 * np.abs(d)[:, None] * (1 - 1e-6)
    assert np.all(err[inside] <= (np.abs(d)[:, None] * (0.5 + 1e-6)).repeat(32, 1)[inside])
    clipped = ~inside & (np.sign(wb) == -np.sign(m)[:, None])
    assert np.all(codes[clipped] == 15)
    return buf


def check_q80_quantizer(lib, w):
    """Q8_0: the activation rule applied to weight blocks (the hand-pinned activation
    quantizer gives the same codes and scales), so |w - d q| <= d / 2 and the
    largest-magnitude weight gets +-127."""
    rows, cols = w.shape
    buf = oracle.quantize_q80(w, lib=lib)
    n = rows * cols // 32
    xq, xd = oracle.quantize_act(w.reshape(1, -1), lib=lib)
    codes = oracle.q80_codes(buf, rows, cols).reshape(-1)
    scales = oracle.q80_scales(buf, rows, cols).reshape(-1)
    assert np.array_equal(codes, xq.reshape(-1))
    assert np.array_equal(scales.view(np.uint32), xd.reshape(-1).view(np.uint32))
    what = oracle.dequantize("q80", buf, rows, cols, lib=lib).reshape(n, 32)
    wb = w.astype(np.float64).reshape(n, 32)
    assert np.all(np.abs(wb - what) <= scales.astype(np.float64)[:, None] * (0.5 + 1e-5))
    return buf


# --------------------------------------------------------------- the GEMV --
def _quantize_for(lib, wtype, w):
    if wtype == "q6k":
        return oracle.quantize_q6k(w, negate_scales=True, lib=lib)
    return oracle.quantize(wtype, w, lib=lib)


def check_gemv_bruteforce(lib, wtype, w, x, tol=1e-12):
    rows, cols = w.shape
    buf = _quantize_for(lib, wtype, w)
    xq, xd = oracle.quantize_act(x, lib=lib)
    res = oracle.gemv(wtype, buf, rows, cols, xq, xd, partials=True, lib=lib)
    what = oracle.dequantize(wtype, buf, rows, cols, lib=lib)
    ybf = oracle.bruteforce(what, xq, xd, lib=lib)
    xhat = xd.astype(np.float64).repeat(32, axis=1) * xq
    bound = np.abs(xhat) @ np.abs(what).T           # [nvec][rows]
    assert np.allclose(res["bound"], bound, rtol=1e-12, atol=0)
    assert np.all(np.abs(res["y"] - ybf) <= tol * bound), float(
        (np.abs(res["y"] - ybf) / np.maximum(bound, 1e-300)).max())
    if wtype == "q4k":
        assert np.array_equal(res["S"], oracle.block_sums(xq))
    return buf, xq, xd, res


def check_gemv_onehot(lib, wtype, w, cols_to_probe=(0, 17, 255, 256 + 130)):
    rows, cols = w.shape
    buf = _quantize_for(lib, wtype, w)
    what = oracle.dequantize(wtype, buf, rows, cols, lib=lib)
    ns = cols // 16 if wtype == "q6k" else cols // 32
    sub = 16 if wtype == "q6k" else 32
    for k in cols_to_probe:
        if k >= cols:
            continue
        for c in (np.float32(0.75), np.float32(-3.0)):
            x = np.zeros((1, cols), np.float32)
            x[0, k] = c
            xq, xd = oracle.quantize_act(x, lib=lib)
            assert xq[0, k] == (127 if c > 0 else -127) and np.count_nonzero(xq) == 1
            xh = np.float64(xd[0, k // 32]) * xq[0, k]
            res = oracle.gemv(wtype, buf, rows, cols, xq, xd, partials=True, lib=lib)
            assert np.allclose(res["y"][0], what[:, k] * xh, rtol=1e-15, atol=0)
            # partial P: only sub-block k // sub is non-zero, and it is code * qx
            P = res["P"][0]
            j = k // sub
            others = np.delete(P, j, axis=1)
            assert np.all(others == 0)
            codes = []
            nb = cols // 256
            for r in range(rows):
                i = r * nb + k // 256
                if wtype in ("q40", "q80"):
                    n32 = rows * cols // 32
                    img = oracle.q32_get_block(wtype, buf, n32, r * (cols // 32) + k // 32, lib=lib)
                    if wtype == "q40":
                        codes.append(int(oracle.q40_unpack_block(img, lib=lib)[1][k % 32]) - 8)
                    else:
                        codes.append(int(oracle.q80_unpack_block(img, lib=lib)[1][k % 32]))
                elif wtype == "q4k":
                    blk = oracle.q4k_get_block(buf, rows * nb, i, lib=lib)
                    codes.append(int(oracle.q4k_unpack_block(blk, lib=lib)[4][k % 256]))
                else:
                    body, _ = oracle.q6k_get_block(buf, rows * nb, i, lib=lib)
                    codes.append(int(oracle.q6k_unpack_block(body, lib=lib)[1][k % 256]) - 32)
            assert np.array_equal(P[:, j], np.array(codes) * int(xq[0, k]))
            assert ns == P.shape[1]


def check_gemv_special(lib):
    rng = np.random.default_rng(5)
    rows, cols = 6, 512
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    for wtype in ("q4k", "q6k"):
        buf = (oracle.quantize_q4k(w, lib=lib) if wtype == "q4k"
               else oracle.quantize_q6k(w, lib=lib))
        what = oracle.dequantize(wtype, buf, rows, cols, lib=lib)
        # zero input: y = 0 exactly
        xq, xd = oracle.quantize_act(np.zeros((1, cols), np.float32), lib=lib)
        res = oracle.gemv(wtype, buf, rows, cols, xq, xd, lib=lib)
        assert np.all(res["y"] == 0) and np.all(res["bound"] == 0)
        # constant input c: all codes 127, y = xd * 127 * sum of the row
        c = np.float32(0.3)
        xq, xd = oracle.quantize_act(np.full((1, cols), c, np.float32), lib=lib)
        assert np.all(xq == 127)
        res = oracle.gemv(wtype, buf, rows, cols, xq, xd, lib=lib)
        want = np.float64(xd[0, 0]) * 127 * what.sum(axis=1)
        assert np.all(np.abs(res["y"][0] - want) <= 1e-12 * res["bound"][0])
    # Q4_K with every sub-scale 0: y = -sum_j xd_j * dmin * m_j * S_j
    q = np.full(256, 9, np.uint8)
    m = np.arange(8, dtype=np.uint8) * 7 + 3
    blk = oracle.q4k_pack_block(0x3C00, 0x2E66, np.zeros(8, np.uint8), m, q, lib=lib)
    x = rng.standard_normal((1, 256)).astype(np.float32)
    xq, xd = oracle.quantize_act(x, lib=lib)
    S = oracle.block_sums(xq)[0].astype(np.float64)
    dmin = float(np.array([0x2E66], np.uint16).view(np.float16)[0])
    want = -np.sum(xd[0].astype(np.float64) * dmin * m * S)
    got = oracle.gemv("q4k", oracle.q4k_tensor([blk], lib=lib), 1, 256, xq, xd, lib=lib)["y"][0, 0]
    assert abs(got - want) <= 1e-15 * abs(want)
    # Q4_K with dmin = 0: the pure scale path d * sc_j * P_j
    blk = oracle.q4k_pack_block(0x3C00, 0x0000, np.arange(8, dtype=np.uint8) + 1, m,
                                np.arange(256, dtype=np.uint8) % 16, lib=lib)
    res = oracle.gemv("q4k", oracle.q4k_tensor([blk], lib=lib), 1, 256, xq, xd, partials=True,
                      lib=lib)
    want = np.sum(xd[0].astype(np.float64) * (np.arange(8) + 1) * res["P"][0, 0])
    assert abs(res["y"][0, 0] - want) <= 1e-15 * abs(want)
    # Q6_K with every code 32: P = 0 and y = 0 exactly
    body = oracle.q6k_pack_block(np.full(16, 77, np.int8), np.full(256, 32, np.uint8), lib=lib)
    tensor = oracle.q6k_tensor([body], [0x3C00], lib=lib)
    res = oracle.gemv("q6k", tensor, 1, 256, xq, xd, partials=True, lib=lib)
    assert np.all(res["P"] == 0) and res["y"][0, 0] == 0.0


def check_gemv_extremes(lib):
    cols = 512
    x_pos = np.full((1, cols), 2.0, np.float32)
    x_neg = np.full((1, cols), -2.0, np.float32)
    # Q4_K: every code 15 against every activation code 127: P = 15 * 127 * 32 = 60960
    blk = oracle.q4k_pack_block(0x3C00, 0x3C00, np.full(8, 63, np.uint8), np.full(8, 63, np.uint8),
                                np.full(256, 15, np.uint8), lib=lib)
    buf = oracle.q4k_tensor([blk, blk], lib=lib)
    xq, xd = oracle.quantize_act(x_pos, lib=lib)
    res = oracle.gemv("q4k", buf, 1, cols, xq, xd, partials=True, lib=lib)
    assert np.all(res["P"] == 60960) and np.all(res["S"] == 127 * 32)
    # Q6_K: every code 0 (value -32) against every activation code -127: P = 32 * 127 * 16 = 65024
    body = oracle.q6k_pack_block(np.full(16, -128, np.int8), np.zeros(256, np.uint8), lib=lib)
    tensor = oracle.q6k_tensor([body, body], [0x3C00] * 2, lib=lib)
    xq, xd = oracle.quantize_act(x_neg, lib=lib)
    res = oracle.gemv("q6k", tensor, 1, cols, xq, xd, partials=True, lib=lib)
    assert np.all(res["P"] == 65024)
    what = oracle.dequantize("q6k", tensor, 1, cols, lib=lib)
    assert np.all(what == 1.0 * -128 * -32)
    # Q8_0: every code 127 against every activation code 127: P = 127 * 127 * 32 = 516128
    img = oracle.q80_pack_block(np.float32(1.0), np.full(32, 127, np.int8), lib=lib)
    tensor = oracle.q32_tensor("q80", [img] * (cols // 32), lib=lib)
    xq, xd = oracle.quantize_act(x_pos, lib=lib)
    res = oracle.gemv("q80", tensor, 1, cols, xq, xd, partials=True, lib=lib)
    assert np.all(res["P"] == 516128)
    # Q4_0: every code 0 (value -8) against -127: P = 8 * 127 * 32 = 32512; code 15 gives
    # 7 * -127 * 32 = -28448
    img0 = oracle.q40_pack_block(0x3C00, np.zeros(32, np.uint8), lib=lib)
    img15 = oracle.q40_pack_block(0x3C00, np.full(32, 15, np.uint8), lib=lib)
    tensor = oracle.q32_tensor("q40", [img0, img15] * (cols // 64), lib=lib)
    xq, xd = oracle.quantize_act(x_neg, lib=lib)
    res = oracle.gemv("q40", tensor, 1, cols, xq, xd, partials=True, lib=lib)
    assert np.all(res["P"][0, 0, 0::2] == 32512) and np.all(res["P"][0, 0, 1::2] == -28448)
