"""CPU oracle for the block-quantized GEMV (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The GPU library never imports it and shares no code with it.

Thin ctypes binding over `qgemv_oracle.c` (plain C, float64 results, exact
integer partials). The arithmetic lives in the C file; this module only moves
numpy arrays in and out. `build()` compiles the C file with gcc into
`oracle/_build/liboracle.so`; loading builds it when it is missing.

Byte layouts (restated in the C file). N = rows * cols/256 super-blocks, block i = r*cols/256 + b:
  Q4_K tensor  = codes plane (128 bytes per block) then header plane (16 bytes per block);
                 one block's "image" is its 16 header bytes followed by its 128 code bytes.
  Q6_K tensor  = low-bit plane (128), high-bit plane (64), scale plane (16), d plane (2 bytes
                 per block); one block's "body" is its low bits, high bits and scales (208 bytes).
  Q4_0 tensor  = codes plane (16 bytes per 32-weight block) then fp16 scale plane (2 bytes);
                 one block's "image" is its fp16 d followed by its 16 code bytes.
  Q8_0 tensor  = two codes planes (int8 codes 0..15, then codes 16..31 of each block, 16
                 bytes per block each) then float32 scale plane (4 bytes); the image is d
                 followed by the 32 codes.
  activations  = int8 codes [nvec][cols] and float32 scales [nvec][cols/32].
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qgemv_oracle.c")
_LIB = os.path.join(_HERE, "_build", "liboracle.so")

Q4K_BYTES = 144
Q6K_BODY = 208
Q6K_BYTES = 210
QK = 256
QB = 32              # weights per Q4_0 / Q8_0 block
Q40_BYTES = 18
Q80_BYTES = 36
WTYPES = ("q4k", "q6k", "q40", "q80")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra"]

_lock = threading.Lock()
_lib = None


def build(out: str = _LIB, extra_flags=(), src: str = _SRC) -> str:
    """Compile the oracle with gcc (always rebuilds). Returns the library path."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra_flags, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _p(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype)) if a is not None else None


def load(path: str | None = None):
    """Load the compiled oracle (building it first if it is missing)."""
    global _lib
    with _lock:
        if path is None and _lib is not None:
            return _lib
        lib_path = path or _LIB
        if not os.path.exists(lib_path):
            build(lib_path)
        lib = ctypes.CDLL(lib_path)
        u8p, i8p, u16p = (ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(ctypes.c_int8),
                          ctypes.POINTER(ctypes.c_uint16))
        f32p, f64p, i32p = (ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double),
                            ctypes.POINTER(ctypes.c_int32))
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        sig = {
            "orc_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
            "orc_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
            "orc_f32_to_f16_array": (None, [f32p, u16p, i64]),
            "orc_f16_to_f32_array": (None, [u16p, f32p, i64]),
            "orc_quantize_act": (None, [f32p, i64, i32, i8p, f32p]),
            "orc_q4k_pack_block": (None, [ctypes.c_uint16, ctypes.c_uint16, u8p, u8p, u8p, u8p]),
            "orc_q4k_unpack_block": (None, [u8p, u16p, u16p, u8p, u8p, u8p]),
            "orc_q6k_pack_block": (None, [i8p, u8p, u8p]),
            "orc_q6k_unpack_block": (None, [u8p, i8p, u8p]),
            "orc_quantize_q4k": (None, [f32p, i64, i64, u8p]),
            "orc_quantize_q6k": (None, [f32p, i64, i64, u8p, ctypes.c_int]),
            "orc_dequant_q4k": (None, [u8p, i64, i64, f64p]),
            "orc_dequant_q6k": (None, [u8p, i64, i64, f64p]),
            "orc_gemv_q4k": (None, [u8p, i64, i64, i32, i8p, f32p, i32p, i32p, f64p, f64p]),
            "orc_gemv_q6k": (None, [u8p, i64, i64, i32, i8p, f32p, i32p, f64p, f64p]),
            "orc_q4k_get_block": (None, [u8p, i64, i64, u8p]),
            "orc_q4k_put_block": (None, [u8p, i64, i64, u8p]),
            "orc_q6k_get_block": (None, [u8p, i64, i64, u8p, u16p]),
            "orc_q6k_put_block": (None, [u8p, i64, i64, u8p, ctypes.c_uint16]),
            "orc_bruteforce": (None, [f64p, i64, i64, i32, i8p, f32p, f64p]),
            "orc_q40_pack_block": (None, [ctypes.c_uint16, u8p, u8p]),
            "orc_q40_unpack_block": (None, [u8p, u16p, u8p]),
            "orc_q80_pack_block": (None, [ctypes.c_float, i8p, u8p]),
            "orc_q80_unpack_block": (None, [u8p, f32p, i8p]),
            "orc_q40_get_block": (None, [u8p, i64, i64, u8p]),
            "orc_q40_put_block": (None, [u8p, i64, i64, u8p]),
            "orc_q80_get_block": (None, [u8p, i64, i64, u8p]),
            "orc_q80_put_block": (None, [u8p, i64, i64, u8p]),
            "orc_quantize_q40": (None, [f32p, i64, i64, u8p]),
            "orc_quantize_q80": (None, [f32p, i64, i64, u8p]),
            "orc_dequant_q40": (None, [u8p, i64, i64, f64p]),
            "orc_dequant_q80": (None, [u8p, i64, i64, f64p]),
            "orc_gemv_q40": (None, [u8p, i64, i64, i32, i8p, f32p, i32p, f64p, f64p]),
            "orc_gemv_q80": (None, [u8p, i64, i64, i32, i8p, f32p, i32p, f64p, f64p]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _lib = lib
        return lib


# ------------------------------------------------------------------ fp16 --
def f32_to_f16(x, lib=None) -> np.ndarray:
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.orc_f32_to_f16_array(_p(x, ctypes.c_float), _p(out, ctypes.c_uint16), x.size)
    return out


def f16_to_f32(h, lib=None) -> np.ndarray:
    lib = lib or load()
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib.orc_f16_to_f32_array(_p(h, ctypes.c_uint16), _p(out, ctypes.c_float), h.size)
    return out


# ----------------------------------------------------------- activations --
def quantize_act(x, lib=None):
    """x float32 [nvec][cols] -> (xq int8 [nvec][cols], xd float32 [nvec][cols/32])."""
    lib = lib or load()
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
    nvec, cols = x.shape
    xq = np.empty((nvec, cols), dtype=np.int8)
    xd = np.empty((nvec, cols // 32), dtype=np.float32)
    lib.orc_quantize_act(_p(x, ctypes.c_float), cols, nvec, _p(xq, ctypes.c_int8),
                         _p(xd, ctypes.c_float))
    return xq, xd


# ---------------------------------------------------------- block layout --
def q4k_pack_block(d16: int, dmin16: int, sc, m, q, lib=None) -> np.ndarray:
    lib = lib or load()
    sc = np.ascontiguousarray(sc, dtype=np.uint8)
    m = np.ascontiguousarray(m, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.empty(Q4K_BYTES, dtype=np.uint8)
    lib.orc_q4k_pack_block(d16, dmin16, _p(sc, ctypes.c_uint8), _p(m, ctypes.c_uint8),
                           _p(q, ctypes.c_uint8), _p(out, ctypes.c_uint8))
    return out


def q4k_unpack_block(blk, lib=None):
    """-> (d fp16 bits, dmin fp16 bits, sc[8], m[8], q[256])"""
    lib = lib or load()
    blk = np.ascontiguousarray(blk, dtype=np.uint8)
    d = np.zeros(1, np.uint16)
    dm = np.zeros(1, np.uint16)
    sc = np.zeros(8, np.uint8)
    m = np.zeros(8, np.uint8)
    q = np.zeros(QK, np.uint8)
    lib.orc_q4k_unpack_block(_p(blk, ctypes.c_uint8), _p(d, ctypes.c_uint16),
                             _p(dm, ctypes.c_uint16), _p(sc, ctypes.c_uint8),
                             _p(m, ctypes.c_uint8), _p(q, ctypes.c_uint8))
    return int(d[0]), int(dm[0]), sc, m, q


def q6k_pack_block(sc, q, lib=None) -> np.ndarray:
    lib = lib or load()
    sc = np.ascontiguousarray(sc, dtype=np.int8)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.empty(Q6K_BODY, dtype=np.uint8)
    lib.orc_q6k_pack_block(_p(sc, ctypes.c_int8), _p(q, ctypes.c_uint8), _p(out, ctypes.c_uint8))
    return out


def q6k_unpack_block(body, lib=None):
    """-> (sc int8[16], q uint8[256])"""
    lib = lib or load()
    body = np.ascontiguousarray(body, dtype=np.uint8)
    sc = np.zeros(16, np.int8)
    q = np.zeros(QK, np.uint8)
    lib.orc_q6k_unpack_block(_p(body, ctypes.c_uint8), _p(sc, ctypes.c_int8),
                             _p(q, ctypes.c_uint8))
    return sc, q


def tensor_bytes(wtype: str, rows: int, cols: int) -> int:
    if wtype in ("q40", "q80"):
        return rows * (cols // QB) * (Q40_BYTES if wtype == "q40" else Q80_BYTES)
    return rows * (cols // QK) * (Q4K_BYTES if wtype == "q4k" else Q6K_BYTES)


def q40_pack_block(d16: int, q, lib=None) -> np.ndarray:
    """18-byte Q4_0 image from fp16 bits of d and 32 codes in [0, 15]."""
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.empty(Q40_BYTES, dtype=np.uint8)
    lib.orc_q40_pack_block(int(d16), _p(q, ctypes.c_uint8), _p(out, ctypes.c_uint8))
    return out


def q40_unpack_block(img, lib=None):
    """-> (fp16 bits of d, q uint8[32])"""
    lib = lib or load()
    img = np.ascontiguousarray(img, dtype=np.uint8)
    d = np.zeros(1, np.uint16)
    q = np.zeros(QB, np.uint8)
    lib.orc_q40_unpack_block(_p(img, ctypes.c_uint8), _p(d, ctypes.c_uint16), _p(q, ctypes.c_uint8))
    return int(d[0]), q


def q80_pack_block(d: float, q, lib=None) -> np.ndarray:
    """36-byte Q8_0 image from a float32 d and 32 int8 codes."""
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.int8)
    out = np.empty(Q80_BYTES, dtype=np.uint8)
    lib.orc_q80_pack_block(float(d), _p(q, ctypes.c_int8), _p(out, ctypes.c_uint8))
    return out


def q80_unpack_block(img, lib=None):
    """-> (d float32, q int8[32])"""
    lib = lib or load()
    img = np.ascontiguousarray(img, dtype=np.uint8)
    d = np.zeros(1, np.float32)
    q = np.zeros(QB, np.int8)
    lib.orc_q80_unpack_block(_p(img, ctypes.c_uint8), _p(d, ctypes.c_float), _p(q, ctypes.c_int8))
    return np.float32(d[0]), q


def q32_get_block(wtype: str, buf, nblocks: int, i: int, lib=None) -> np.ndarray:
    """The image of block i of a Q4_0 / Q8_0 tensor of nblocks blocks."""
    lib = lib or load()
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    size = Q40_BYTES if wtype == "q40" else Q80_BYTES
    assert buf.size == nblocks * size
    img = np.empty(size, dtype=np.uint8)
    fn = lib.orc_q40_get_block if wtype == "q40" else lib.orc_q80_get_block
    fn(_p(buf, ctypes.c_uint8), nblocks, i, _p(img, ctypes.c_uint8))
    return img


def q32_tensor(wtype: str, images, lib=None) -> np.ndarray:
    """A Q4_0 / Q8_0 tensor from a list of block images (block i = images[i])."""
    lib = lib or load()
    n = len(images)
    size = Q40_BYTES if wtype == "q40" else Q80_BYTES
    out = np.zeros(n * size, dtype=np.uint8)
    fn = lib.orc_q40_put_block if wtype == "q40" else lib.orc_q80_put_block
    for i, img in enumerate(images):
        img = np.ascontiguousarray(img, dtype=np.uint8)
        fn(_p(out, ctypes.c_uint8), n, i, _p(img, ctypes.c_uint8))
    return out


def q4k_get_block(buf, nblocks: int, i: int, lib=None) -> np.ndarray:
    """The 144-byte image (header, codes) of block i of a Q4_K tensor of nblocks blocks."""
    lib = lib or load()
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    assert buf.size == nblocks * Q4K_BYTES
    img = np.empty(Q4K_BYTES, dtype=np.uint8)
    lib.orc_q4k_get_block(_p(buf, ctypes.c_uint8), nblocks, i, _p(img, ctypes.c_uint8))
    return img


def q4k_tensor(images, lib=None) -> np.ndarray:
    """A Q4_K tensor from a list of 144-byte block images (block i = images[i])."""
    lib = lib or load()
    n = len(images)
    out = np.zeros(n * Q4K_BYTES, dtype=np.uint8)
    for i, img in enumerate(images):
        img = np.ascontiguousarray(img, dtype=np.uint8)
        lib.orc_q4k_put_block(_p(out, ctypes.c_uint8), n, i, _p(img, ctypes.c_uint8))
    return out


def q6k_get_block(buf, nblocks: int, i: int, lib=None):
    """(208-byte body, fp16 bits of d) of block i of a Q6_K tensor of nblocks blocks."""
    lib = lib or load()
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    assert buf.size == nblocks * Q6K_BYTES
    body = np.empty(Q6K_BODY, dtype=np.uint8)
    d = np.zeros(1, dtype=np.uint16)
    lib.orc_q6k_get_block(_p(buf, ctypes.c_uint8), nblocks, i, _p(body, ctypes.c_uint8),
                          _p(d, ctypes.c_uint16))
    return body, int(d[0])


def q6k_tensor(bodies, d16s, lib=None) -> np.ndarray:
    """A Q6_K tensor from lists of 208-byte bodies and fp16 bits of d (block i = index i)."""
    lib = lib or load()
    n = len(bodies)
    out = np.zeros(n * Q6K_BYTES, dtype=np.uint8)
    for i, (body, d) in enumerate(zip(bodies, d16s)):
        body = np.ascontiguousarray(body, dtype=np.uint8)
        lib.orc_q6k_put_block(_p(out, ctypes.c_uint8), n, i, _p(body, ctypes.c_uint8), int(d))
    return out


def blocks_of(wtype: str, buf, rows: int, cols: int, lib=None):
    """All blocks of a tensor: Q4_K -> [N][144] images; Q6_K -> ([N][208] bodies, [N] d bits)."""
    n = rows * (cols // QK)
    if wtype == "q4k":
        return np.stack([q4k_get_block(buf, n, i, lib=lib) for i in range(n)])
    got = [q6k_get_block(buf, n, i, lib=lib) for i in range(n)]
    return np.stack([g[0] for g in got]), np.array([g[1] for g in got], dtype=np.uint16)


# ------------------------------------------------------ weight quantizers --
def quantize_q4k(w, lib=None) -> np.ndarray:
    """w float32 [rows][cols] -> Q4_K tensor, uint8 [rows * cols/256 * 144]."""
    lib = lib or load()
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    out = np.empty(rows * (cols // QK) * Q4K_BYTES, dtype=np.uint8)
    lib.orc_quantize_q4k(_p(w, ctypes.c_float), rows, cols, _p(out, ctypes.c_uint8))
    return out


def quantize_q40(w, lib=None) -> np.ndarray:
    """w float32 [rows][cols] -> Q4_0 tensor, uint8 [rows * cols/32 * 18] (two planes)."""
    lib = lib or load()
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    out = np.empty(rows * (cols // QB) * Q40_BYTES, dtype=np.uint8)
    lib.orc_quantize_q40(_p(w, ctypes.c_float), rows, cols, _p(out, ctypes.c_uint8))
    return out


def quantize_q80(w, lib=None) -> np.ndarray:
    """w float32 [rows][cols] -> Q8_0 tensor, uint8 [rows * cols/32 * 36] (two planes)."""
    lib = lib or load()
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    out = np.empty(rows * (cols // QB) * Q80_BYTES, dtype=np.uint8)
    lib.orc_quantize_q80(_p(w, ctypes.c_float), rows, cols, _p(out, ctypes.c_uint8))
    return out


def quantize(wtype: str, w, lib=None) -> np.ndarray:
    """Any of the four formats (Q6_K with its plain encoding)."""
    return {"q4k": quantize_q4k, "q6k": quantize_q6k, "q40": quantize_q40,
            "q80": quantize_q80}[wtype](w, lib=lib)


def quantize_q6k(w, negate_scales: bool = False, lib=None) -> np.ndarray:
    """w float32 [rows][cols] -> Q6_K tensor, uint8 [rows * cols/256 * 210] (four planes)."""
    lib = lib or load()
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    out = np.empty(rows * (cols // QK) * Q6K_BYTES, dtype=np.uint8)
    lib.orc_quantize_q6k(_p(w, ctypes.c_float), rows, cols, _p(out, ctypes.c_uint8),
                         int(bool(negate_scales)))
    return out


def dequantize(wtype: str, wbuf, rows: int, cols: int, lib=None) -> np.ndarray:
    """Dequantized weights, float64 [rows][cols]."""
    lib = lib or load()
    out = np.empty((rows, cols), dtype=np.float64)
    wbuf = np.ascontiguousarray(wbuf, dtype=np.uint8).reshape(-1)
    if wbuf.size != tensor_bytes(wtype, rows, cols):
        raise ValueError("tensor has %d bytes, expected %d" % (wbuf.size, tensor_bytes(wtype, rows, cols)))
    fn = {"q4k": lib.orc_dequant_q4k, "q6k": lib.orc_dequant_q6k, "q40": lib.orc_dequant_q40,
          "q80": lib.orc_dequant_q80}[wtype]
    fn(_p(wbuf, ctypes.c_uint8), rows, cols, _p(out, ctypes.c_double))
    return out


# ---------------------------------------------------------- integer GEMV --
def gemv(wtype: str, wbuf, rows: int, cols: int, xq, xd, partials: bool = False,
         bound: bool = True, lib=None) -> dict:
    """Integer-formulated GEMV. Returns y [nvec][rows] (float64), bound, and optionally
    the exact partials P (Q4_K, Q4_0, Q8_0 [nvec][rows][cols/32], Q6_K [nvec][rows][cols/16])
    and S [nvec][cols/32] (Q4_K only)."""
    lib = lib or load()
    xq = np.ascontiguousarray(np.atleast_2d(xq), dtype=np.int8)
    xd = np.ascontiguousarray(np.atleast_2d(xd), dtype=np.float32)
    nvec = xq.shape[0]
    if xq.shape != (nvec, cols) or xd.shape != (nvec, cols // 32):
        raise ValueError("activation shapes do not match cols")
    y = np.empty((nvec, rows), dtype=np.float64)
    bnd = np.empty((nvec, rows), dtype=np.float64) if bound else None
    out = {"y": y}
    wbuf = np.ascontiguousarray(wbuf, dtype=np.uint8).reshape(-1)
    if wbuf.size != tensor_bytes(wtype, rows, cols):
        raise ValueError("tensor has %d bytes, expected %d" % (wbuf.size, tensor_bytes(wtype, rows, cols)))
    if wtype == "q4k":
        P = np.empty((nvec, rows, cols // 32), dtype=np.int32) if partials else None
        S = np.empty((nvec, cols // 32), dtype=np.int32) if partials else None
        lib.orc_gemv_q4k(_p(wbuf, ctypes.c_uint8), rows, cols, nvec, _p(xq, ctypes.c_int8),
                         _p(xd, ctypes.c_float), _p(P, ctypes.c_int32), _p(S, ctypes.c_int32),
                         _p(y, ctypes.c_double), _p(bnd, ctypes.c_double))
        if partials:
            out["P"], out["S"] = P, S
    elif wtype == "q6k":
        P = np.empty((nvec, rows, cols // 16), dtype=np.int32) if partials else None
        lib.orc_gemv_q6k(_p(wbuf, ctypes.c_uint8), rows, cols, nvec, _p(xq, ctypes.c_int8),
                         _p(xd, ctypes.c_float), _p(P, ctypes.c_int32), _p(y, ctypes.c_double),
                         _p(bnd, ctypes.c_double))
        if partials:
            out["P"] = P
    elif wtype in ("q40", "q80"):
        P = np.empty((nvec, rows, cols // 32), dtype=np.int32) if partials else None
        fn = lib.orc_gemv_q40 if wtype == "q40" else lib.orc_gemv_q80
        fn(_p(wbuf, ctypes.c_uint8), rows, cols, nvec, _p(xq, ctypes.c_int8),
           _p(xd, ctypes.c_float), _p(P, ctypes.c_int32), _p(y, ctypes.c_double),
           _p(bnd, ctypes.c_double))
        if partials:
            out["P"] = P
    else:
        raise ValueError("unknown weight type %r" % wtype)
    if bound:
        out["bound"] = bnd
    return out


def block_sums(xq) -> np.ndarray:
    """S [nvec][cols/32]: exact sums of the activation codes per block of 32 (Q4_K's S)."""
    xq = np.atleast_2d(np.asarray(xq, dtype=np.int64))
    nvec, cols = xq.shape
    return xq.reshape(nvec, cols // 32, 32).sum(axis=2).astype(np.int32)


def bruteforce(what, xq, xd, lib=None) -> np.ndarray:
    """y [nvec][rows] = what @ (xd * xq) in float64, from a dequantized matrix."""
    lib = lib or load()
    what = np.ascontiguousarray(what, dtype=np.float64)
    xq = np.ascontiguousarray(np.atleast_2d(xq), dtype=np.int8)
    xd = np.ascontiguousarray(np.atleast_2d(xd), dtype=np.float32)
    rows, cols = what.shape
    nvec = xq.shape[0]
    y = np.empty((nvec, rows), dtype=np.float64)
    lib.orc_bruteforce(_p(what, ctypes.c_double), rows, cols, nvec, _p(xq, ctypes.c_int8),
                       _p(xd, ctypes.c_float), _p(y, ctypes.c_double))
    return y


def planes(wtype: str, wbuf, rows: int, cols: int) -> list:
    """The planes of a tensor as [rows][bytes per row] views (Q4_K: codes, headers; Q6_K: low
    bits, high bits, scales, d; Q4_0: codes, scales; Q8_0: codes 0..15 of each block, codes
    16..31, scales)."""
    nb = cols // (QB if wtype in ("q40", "q80") else QK)
    n = rows * nb
    wbuf = np.ascontiguousarray(wbuf, dtype=np.uint8).reshape(-1)
    widths = {"q4k": [128, 16], "q6k": [128, 64, 16, 2], "q40": [16, 2], "q80": [16, 16, 4]}[wtype]
    out, off = [], 0
    for wdt in widths:
        out.append(wbuf[off:off + n * wdt].reshape(rows, nb * wdt))
        off += n * wdt
    return out


def q80_codes(wbuf, rows: int, cols: int) -> np.ndarray:
    """The int8 codes of a Q8_0 tensor as [rows][cols], from its two codes planes."""
    lo, hi, _ = planes("q80", wbuf, rows, cols)
    n = rows * (cols // QB)
    return np.concatenate([lo.reshape(n, 16), hi.reshape(n, 16)], axis=1).reshape(
        rows, cols).view(np.int8)


def q80_scales(wbuf, rows: int, cols: int) -> np.ndarray:
    """The float32 scales of a Q8_0 tensor as [rows][cols/32]."""
    return planes("q80", wbuf, rows, cols)[2].copy().view(np.float32)


def from_planes(parts) -> np.ndarray:
    return np.concatenate([np.ascontiguousarray(p).reshape(-1) for p in parts])


def row_slice(wtype: str, wbuf, rows: int, cols: int, r0: int, r1: int) -> np.ndarray:
    """The tensor of rows r0 .. r1 - 1 of a quantized tensor, in the same format."""
    return from_planes([p[r0:r1] for p in planes(wtype, wbuf, rows, cols)])


def concat_rows(wtype: str, parts, cols: int) -> np.ndarray:
    """One tensor from tensors of consecutive row ranges [(buf, rows), ...]."""
    per = [planes(wtype, b, r, cols) for b, r in parts]
    return from_planes([np.concatenate([p[k] for p in per]) for k in range(len(per[0]))])


def gemv_threaded(wtype: str, wbuf, rows: int, cols: int, xq, xd, threads: int) -> np.ndarray:
    """The same integer GEMV over equal contiguous row ranges on `threads` host threads
    (ctypes releases the GIL during each call). Returns y only."""
    if threads <= 1:
        return gemv(wtype, wbuf, rows, cols, xq, xd, bound=False)["y"]
    nvec = np.atleast_2d(xq).shape[0]
    y = np.empty((nvec, rows), dtype=np.float64)
    cuts = [rows * i // threads for i in range(threads + 1)]
    parts = [row_slice(wtype, wbuf, rows, cols, cuts[i], cuts[i + 1]) for i in range(threads)]

    def work(i):
        r0, r1 = cuts[i], cuts[i + 1]
        if r1 > r0:
            y[:, r0:r1] = gemv(wtype, parts[i], r1 - r0, cols, xq, xd, bound=False)["y"]

    ts = [threading.Thread(target=work, args=(i,)) for i in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    return y
