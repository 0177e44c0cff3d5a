"""Seeded synthetic inputs for the block-quantized GEMV: random numbers only.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It draws Gaussian weights and activations and picks outlier rows; it
holds none of the method's arithmetic (no quantization, no dot products).

Generator: splitmix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), used as a counter-based stream:
output number k (k = 0, 1, ...) of a seed s is mix64(s + (k + 1) * GOLDEN),
so any slice of a stream can be drawn without drawing what precedes it.

Uniforms take the top 53 bits of an output, mapped into (0, 1]. Normals come
from the Box-Muller transform in float64: uniform pair (u1, u2) number p gives
stream elements 2p (radius * cos) and 2p + 1 (radius * sin), with
radius = sqrt(-2 ln u1) and angle 2*pi*u2. They are scaled by sigma in float64
and rounded to float32 (round to nearest even).

Workloads (weights N(0, 0.02), activations N(0, 1)) follow the shapes the
oxinfer README ("Performance") and the genie-ai-runtime post ("The decode arc")
describe as the decode path: one matrix-vector product per linear layer per
generated token, with the vocabulary projection of Gemma 4 E2B (262144 x 1536)
as the largest one.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, counters: np.ndarray) -> np.ndarray:
    """Outputs number `counters` (uint64 array) of the splitmix64 stream of `seed`."""
    k = np.asarray(counters, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + (k + np.uint64(1)) * GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform01(seed: int, counters: np.ndarray) -> np.ndarray:
    """Uniform float64 in (0, 1] from the top 53 bits of each output."""
    z = splitmix64(seed, counters)
    # 53-bit integers convert to float64 exactly (the int64 route is the fast one in numpy)
    top = (z >> np.uint64(11)).astype(np.int64).astype(np.float64)
    return (top + 1.0) * (1.0 / 9007199254740992.0)


_PIECE = 1 << 21   # stream elements per worker task


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_f32(seed: int, start: int, count: int, sigma: float) -> np.ndarray:
    """Elements [start, start + count) of the N(0, sigma^2) float32 stream of `seed`."""
    if count <= 0:
        return np.zeros(0, dtype=np.float32)
    if count > 2 * _PIECE:
        # numpy's float64 trigonometry runs per element; split the range over threads
        # (ufuncs release the GIL). The pieces are cut at even offsets so that no
        # Box-Muller pair is split, which keeps the result identical to one call.
        out = np.empty(count, dtype=np.float32)
        cuts = list(range(start, start + count, _PIECE)) + [start + count]
        cuts = [cuts[0]] + [c - (c % 2) for c in cuts[1:-1]] + [cuts[-1]]

        def fill(i):
            a, b = cuts[i], cuts[i + 1]
            out[a - start:b - start] = _normal_f32_serial(seed, a, b - a, sigma)

        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(len(cuts) - 1)))
        return out
    return _normal_f32_serial(seed, start, count, sigma)


def _normal_f32_serial(seed: int, start: int, count: int, sigma: float) -> np.ndarray:
    p0 = start // 2
    p1 = (start + count + 1) // 2
    pairs = np.arange(p0, p1, dtype=np.uint64)
    u1 = uniform01(seed, pairs * np.uint64(2))
    u2 = uniform01(seed, pairs * np.uint64(2) + np.uint64(1))
    radius = np.sqrt(-2.0 * np.log(u1))
    angle = (2.0 * np.pi) * u2
    z = np.empty(2 * pairs.size, dtype=np.float64)
    z[0::2] = radius * np.cos(angle)
    z[1::2] = radius * np.sin(angle)
    off = start - 2 * p0
    return (z[off:off + count] * sigma).astype(np.float32)


def choose_rows(seed: int, rows: int, count: int) -> np.ndarray:
    """`count` distinct rows of range(rows), uniformly without replacement, sorted.

    Partial Fisher-Yates shuffle: step i swaps position i with position
    i + (output i mod (rows - i)).
    """
    count = min(count, rows)
    perm = np.arange(rows, dtype=np.int64)
    draws = splitmix64(seed, np.arange(count, dtype=np.uint64))
    for i in range(count):
        j = i + int(draws[i] % np.uint64(rows - i))
        perm[i], perm[j] = perm[j], perm[i]
    return np.sort(perm[:count])


@dataclasses.dataclass(frozen=True)
class Workload:
    """One GEMV problem: a weight matrix in one block format and nvec activation vectors."""

    name: str
    wtype: str          # "q4k" or "q6k"
    rows: int
    cols: int
    nvec: int
    seed_w: int
    seed_x: int         # vector v uses seed_x + v
    sigma_w: float = 0.02
    sigma_x: float = 1.0
    outlier_frac: float = 0.0   # fraction of rows scaled by outlier_gain before quantization
    outlier_gain: float = 10.0
    seed_rows: int = 0

    def outlier_rows(self) -> np.ndarray:
        n = int(round(self.outlier_frac * self.rows))
        if n == 0:
            return np.zeros(0, dtype=np.int64)
        return choose_rows(self.seed_rows, self.rows, n)

    def weight_rows(self, row_idx) -> np.ndarray:
        """float32 [len(row_idx)][cols] weights for the given rows (stream element r*cols + c)."""
        row_idx = np.asarray(row_idx, dtype=np.int64).reshape(-1)
        out = np.empty((row_idx.size, self.cols), dtype=np.float32)
        # contiguous runs are drawn in one call
        i = 0
        while i < row_idx.size:
            j = i + 1
            while j < row_idx.size and row_idx[j] == row_idx[j - 1] + 1:
                j += 1
            r0 = int(row_idx[i])
            out[i:j] = normal_f32(self.seed_w, r0 * self.cols, (j - i) * self.cols,
                                  self.sigma_w).reshape(j - i, self.cols)
            i = j
        if self.outlier_frac > 0:
            hot = np.isin(row_idx, self.outlier_rows())
            out[hot] *= np.float32(self.outlier_gain)
        return out

    def weight_block(self, r0: int, r1: int) -> np.ndarray:
        """float32 [r1 - r0][cols] weights of rows r0 .. r1 - 1."""
        return self.weight_rows(np.arange(r0, r1, dtype=np.int64))

    def activations(self) -> np.ndarray:
        """float32 [nvec][cols] activation vectors."""
        return np.stack([normal_f32(self.seed_x + v, 0, self.cols, self.sigma_x)
                         for v in range(self.nvec)])


# The decode workloads. Index i uses weight seed 1000 + i, activation seed 2000 + 100 i (+ v),
# row seed 3000 + i.
WORKLOADS = {
    "q4k_512x512": Workload("q4k_512x512", "q4k", 512, 512, 1, 1000, 2000),
    "q4k_8192x2048": Workload("q4k_8192x2048", "q4k", 8192, 2048, 1, 1001, 2100),
    "q6k_2048x8192": Workload("q6k_2048x8192", "q6k", 2048, 8192, 1, 1002, 2200),
    "q4k_262144x1536": Workload("q4k_262144x1536", "q4k", 262144, 1536, 1, 1003, 2300,
                                outlier_frac=0.01, seed_rows=3003),
    "q4k_16384x2048_b8": Workload("q4k_16384x2048_b8", "q4k", 16384, 2048, 8, 1004, 2400),
    # the 32-weight formats at the vocabulary-projection shape (weight seeds 1005, 1006)
    "q40_262144x1536": Workload("q40_262144x1536", "q40", 262144, 1536, 1,
                                1005, 2700, outlier_frac=0.01, seed_rows=3005),
    "q80_262144x1536": Workload("q80_262144x1536", "q80", 262144, 1536, 1, 1006, 2800,
                                outlier_frac=0.01, seed_rows=3006),
    # ... and Q6_K there (the format a vocabulary projection is often kept in; weight seed 1009)
    "q6k_262144x1536": Workload("q6k_262144x1536", "q6k", 262144, 1536, 1, 1009, 3700,
                                outlier_frac=0.01, seed_rows=3009),
    # a few vectors at once (several sequences decoded together) on the Q4_0 and Q6_K
    # projections above (their weights; vector v has activation seed 3800 + v, resp. 3900 + v)
    "q40_262144x1536_b8": Workload("q40_262144x1536_b8", "q40", 262144, 1536, 8, 1005, 3800,
                                   outlier_frac=0.01, seed_rows=3005),
    "q6k_262144x1536_b8": Workload("q6k_262144x1536_b8", "q6k", 262144, 1536, 8, 1009, 3900,
                                   outlier_frac=0.01, seed_rows=3009),
    # 16 vectors (tokens verified together) on a 65536-row Q4_0 matrix (weight seed 1008;
    # vector v has activation seed 4000 + v)
    "q40_65536x2048_b16": Workload("q40_65536x2048_b16", "q40", 65536, 2048, 16, 1008, 4000),
    # many vectors at once (tokens verified or prefilled together) on the matrices above:
    # vector v has activation seed 3100 + v (resp. 3400 + v)
    "q4k_262144x1536_b64": Workload("q4k_262144x1536_b64", "q4k", 262144, 1536, 64, 1003, 3100,
                                    outlier_frac=0.01, seed_rows=3003),
    "q4k_16384x2048_b64": Workload("q4k_16384x2048_b64", "q4k", 16384, 2048, 64, 1004, 3400),
    # a row wider than one pass of 256 chunks (16384 columns = 512 chunks): the column split
    # with its ordered second pass (weight seed 1007)
    "q4k_4096x16384": Workload("q4k_4096x16384", "q4k", 4096, 16384, 1, 1007, 2900),
}


@dataclasses.dataclass(frozen=True)
class WorkloadGroup:
    """Several weight matrices that multiply the same activation vectors (one multi-matrix
    product). The parts share cols, nvec and the activation seed."""

    name: str
    parts: tuple

    @property
    def cols(self) -> int:
        return self.parts[0].cols

    @property
    def nvec(self) -> int:
        return self.parts[0].nvec

    def activations(self) -> np.ndarray:
        return self.parts[0].activations()


def _group(name, cols, nvec, seed_x, parts):
    return WorkloadGroup(name, tuple(Workload("%s.%s" % (name, p), wtype, rows, cols, nvec, seed_w,
                                              seed_x) for p, wtype, rows, seed_w in parts))


# Multi-matrix workloads: shaped like one decoder layer's projections at width 1536 (the width
# of the 262144 x 1536 projection above), weights N(0, 0.02), x N(0, 1). Weight seeds 1010+,
# activation seeds 2500+.
GROUPS = {
    "qkv_1536": _group("qkv_1536", 1536, 1, 2500, [("q", "q4k", 2048, 1010),
                                                   ("k", "q4k", 512, 1011),
                                                   ("v", "q6k", 512, 1012)]),
    "gate_up_1536": _group("gate_up_1536", 1536, 1, 2600, [("gate", "q4k", 6144, 1013),
                                                           ("up", "q4k", 6144, 1014)]),
}


@dataclasses.dataclass(frozen=True)
class DecodeLayer:
    """The products of one decoder layer for one token, in the order a decode step makes them:
    the attention projections (one multi-matrix product on the normalized hidden state), the
    output projection (on the attention output), the FFN gate and up projections (one
    multi-matrix product) and the down projection (on the gated FFN activation)."""

    qkv: WorkloadGroup
    o: Workload
    gate_up: WorkloadGroup
    down: Workload


@dataclasses.dataclass(frozen=True)
class DecodeStep:
    """One generated token's matrix-vector products: the layers in order, then the vocabulary
    projection. The inputs of the products are independent seeded vectors, standing for the
    outputs of the operations between them (normalization, attention, gating), which are not
    part of this library."""

    name: str
    layers: tuple
    head: Workload

    def products(self):
        """[(kind, item)] in step order: kind "multi" (a WorkloadGroup) or "one" (a Workload)."""
        out = []
        for layer in self.layers:
            out += [("multi", layer.qkv), ("one", layer.o), ("multi", layer.gate_up),
                    ("one", layer.down)]
        out.append(("one", self.head))
        return out


def decode_step(name, layers, hidden, q, kv, ffn, head, formats=("q4k", "q4k", "q6k", "q4k",
                                                                  "q4k", "q4k", "q4k"),
                nvec=1, seed=100000):
    """A decode step of `layers` identical layers at width `hidden`: Q, K, V projections of q,
    kv, kv rows, output projection hidden x q, gate and up ffn x hidden, down hidden x ffn.
    formats: the weight formats of (q, k, v, o, gate, up, down). Layer l's matrix k (in that
    order) has weight seed seed + 16 l + k; its four inputs have seeds seed + 100000 + 100 l +
    10 j (+ v)."""
    fq, fk, fv, fo, fg, fu, fd = formats
    out = []
    for l in range(layers):
        sw = seed + 16 * l
        sx = seed + 100000 + 100 * l
        qkv = WorkloadGroup("%s.l%d.qkv" % (name, l), (
            Workload("%s.l%d.q" % (name, l), fq, q, hidden, nvec, sw + 0, sx),
            Workload("%s.l%d.k" % (name, l), fk, kv, hidden, nvec, sw + 1, sx),
            Workload("%s.l%d.v" % (name, l), fv, kv, hidden, nvec, sw + 2, sx)))
        o = Workload("%s.l%d.o" % (name, l), fo, hidden, q, nvec, sw + 3, sx + 10)
        gu = WorkloadGroup("%s.l%d.gate_up" % (name, l), (
            Workload("%s.l%d.gate" % (name, l), fg, ffn, hidden, nvec, sw + 4, sx + 20),
            Workload("%s.l%d.up" % (name, l), fu, ffn, hidden, nvec, sw + 5, sx + 20)))
        down = Workload("%s.l%d.down" % (name, l), fd, hidden, ffn, nvec, sw + 6, sx + 30)
        out.append(DecodeLayer(qkv, o, gu, down))
    return DecodeStep(name, tuple(out), head)


# A decode step shaped like Gemma 4 E2B, the model of the genie-ai-runtime post and of the
# "Gemma WebGPU Engine" page: 35 layers and the 1536 -> 2048 / 256 / 256 attention projections
# and 2048 -> 1536 output projection of that page ("Roadmap"), an FFN of width 6144 (4 x 1536;
# the pages give no FFN width), the 262144 x 1536 vocabulary projection above as the head; V in
# Q6_K as in the post's triple QKV product ("v1.2.0"), every other matrix Q4_K.
DECODE_STEPS = {
    "decode_step_1536x35": decode_step("decode_step_1536x35", 35, 1536, 2048, 256, 6144,
                                       WORKLOADS["q4k_262144x1536"]),
}
