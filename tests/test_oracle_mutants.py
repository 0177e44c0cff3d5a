"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is the oracle's C source with one plausible mistake written in (a dropped
term, a wrong sign, a swapped index, a different rounding rule). It is compiled on the
CPU into a temporary library and the pin checks of oracle_pins run against it in a
child process; at least one check must fail for every mutant. The shipped oracle
itself must pass all of them (the control case).
"""

import json
import os
import subprocess
import sys

import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "qgemv_oracle.c")

MUTANTS = {
    "q4k_drop_min_term": (
        "acc += scale * (d * sc * (double)checked32(p) - dmin * m * (double)checked32(s));",
        "acc += scale * (d * sc * (double)checked32(p));"),
    "q4k_min_sign": (
        "acc += scale * (d * sc * (double)checked32(p) - dmin * m * (double)checked32(s));",
        "acc += scale * (d * sc * (double)checked32(p) + dmin * m * (double)checked32(s));"),
    "q4k_nibble_swap": (
        "return (blk[16 + 16 * j + t] >> (4 * h)) & 15;",
        "return (blk[16 + 16 * j + t] >> (4 * (1 - h))) & 15;"),
    "q4k_sc_high_from_m": (
        "int hi = (blk[12 + j / 4] >> (2 * (j % 4))) & 3;\n    return lo | (hi << 4);\n}\n\nstatic int q4k_m",
        "int hi = (blk[14 + j / 4] >> (2 * (j % 4))) & 3;\n    return lo | (hi << 4);\n}\n\nstatic int q4k_m"),
    "q4k_act_scale_index": (
        "double scale = dv[col0 / 32];\n                    acc += scale * (d * sc",
        "double scale = dv[(col0 / 32) ^ 1];\n                    acc += scale * (d * sc"),
    "q6k_offset_31": (
        "p += (int64_t)(q6k_q(body, 16 * j + i) - 32) * xv[col0 + i];",
        "p += (int64_t)(q6k_q(body, 16 * j + i) - 31) * xv[col0 + i];"),
    "q6k_high_bits_shift": (
        "int hi = (body[128 + 8 * k + 4 * g + c] >> (2 * s)) & 3;",
        "int hi = (body[128 + 8 * k + 4 * g + c] >> (2 * c)) & 3;"),
    "q6k_scale_unsigned": (
        "static int q6k_sc(const uint8_t *body, int j) { return (int)(int8_t)body[192 + j]; }",
        "static int q6k_sc(const uint8_t *body, int j) { return (int)body[192 + j]; }"),
    "q6k_wrong_sub_block_scale": (
        "int sc = q6k_sc(body, j);\n                    int64_t p = 0;",
        "int sc = q6k_sc(body, j ^ 1);\n                    int64_t p = 0;"),
    "act_round_half_away": (
        "float code = clampf(rintf(prod), -127.0f, 127.0f);",
        "float code = clampf(roundf(prod), -127.0f, 127.0f);"),
    "act_divide_instead": (
        "float prod = xb[i] * inv;",
        "float prod = amax > 0.0f ? xb[i] / scale : 0.0f;"),
    "act_inverse_unguarded": (
        "            if (!(inv <= FLT_MAX)) inv = 0.0f;\n",
        ""),
    "q80_inverse_unguarded": (
        "            if (!(id <= FLT_MAX)) id = 0.0f;\n",
        ""),
    "act_allow_minus_128": (
        "float code = clampf(rintf(prod), -127.0f, 127.0f);",
        "float code = clampf(rintf(prod * 1.004f), -128.0f, 127.0f);"),
    "fp16_subnormal_exponent": (
        "v = ldexpf((float)m, -24);",
        "v = ldexpf((float)m, -25);"),
    "fp16_round_half_up": (
        "if (rest > half || (rest == half && (kept & 1u)))",
        "if (rest >= half)"),
    "q4k_quant_no_offset": (
        "? clampf(rintf((v + off) / step), 0.0f, 15.0f) : 0.0f);",
        "? clampf(rintf((v) / step), 0.0f, 15.0f) : 0.0f);"),
    "q6k_quant_divisor_63": (
        "uint16_t dh = orc_f32_to_f16(smax / 127.0f);\n            float d = orc_f16_to_f32(dh);",
        "uint16_t dh = orc_f32_to_f16(smax / 63.0f);\n            float d = orc_f16_to_f32(dh);"),
    "q40_offset_7": (
        "for (int t = 0; t < QB; t++) c[t] = q40_q(img, t) - 8;",
        "for (int t = 0; t < QB; t++) c[t] = q40_q(img, t) - 7;"),
    "q40_nibble_order": (
        "return t < 16 ? (byte & 15) : (byte >> 4);",
        "return t < 16 ? (byte >> 4) : (byte & 15);"),
    "q40_scale_plane_offset": (
        "memcpy(img, t + 16 * N + 2 * i, 2);",
        "memcpy(img, t + 16 * N + 2 * (i ^ 1), 2);"),
    "q80_scale_from_codes_plane": (
        "memcpy(img, t + 32 * N + 4 * i, 4);",
        "memcpy(img, t + 32 * i, 4);"),
    "q40_quant_scale_sign": (
        "uint16_t dh = m != 0.0f ? orc_f32_to_f16(m / -8.0f) : 0;",
        "uint16_t dh = m != 0.0f ? orc_f32_to_f16(m / 8.0f) : 0;"),
    "q40_quant_divisor_7": (
        "uint16_t dh = m != 0.0f ? orc_f32_to_f16(m / -8.0f) : 0;",
        "uint16_t dh = m != 0.0f ? orc_f32_to_f16(m / -7.0f) : 0;"),
    "q80_quant_divide": (
        "for (int t = 0; t < QB; t++) q[t] = (int8_t)clampf(rintf(wb[t] * id), -127.0f, 127.0f);",
        "for (int t = 0; t < QB; t++) q[t] = (int8_t)clampf(d > 0.0f ? rintf(wb[t] / d) : 0.0f, -127.0f, 127.0f);"),
    # plane order and plane offsets of the Q4_K / Q6_K tensors: a mutant that moves a plane
    # in both the reader and the writer stays self-consistent, so only fixed bytes catch it
    "q4k_header_plane_first": [
        ("memcpy(img, t + 128 * N + 16 * i, 16);\n    memcpy(img + 16, t + 128 * i, 128);",
         "memcpy(img, t + 16 * i, 16);\n    memcpy(img + 16, t + 16 * N + 128 * i, 128);"),
        ("memcpy(t + 128 * N + 16 * i, img, 16);\n    memcpy(t + 128 * i, img + 16, 128);",
         "memcpy(t + 16 * i, img, 16);\n    memcpy(t + 16 * N + 128 * i, img + 16, 128);")],
    "q4k_header_index_read": (
        "memcpy(img, t + 128 * N + 16 * i, 16);",
        "memcpy(img, t + 128 * N + 16 * (N - 1 - i), 16);"),
    "q4k_header_index_both": [
        ("memcpy(img, t + 128 * N + 16 * i, 16);", "memcpy(img, t + 128 * N + 16 * (N - 1 - i), 16);"),
        ("memcpy(t + 128 * N + 16 * i, img, 16);", "memcpy(t + 128 * N + 16 * (N - 1 - i), img, 16);")],
    "q6k_high_and_scale_planes_swapped": [
        ("memcpy(body + 128, t + 128 * N + 64 * i, 64);\n    memcpy(body + 192, t + 192 * N + 16 * i, 16);",
         "memcpy(body + 128, t + 144 * N + 64 * i, 64);\n    memcpy(body + 192, t + 128 * N + 16 * i, 16);"),
        ("memcpy(t + 128 * N + 64 * i, body + 128, 64);\n    memcpy(t + 192 * N + 16 * i, body + 192, 16);",
         "memcpy(t + 144 * N + 64 * i, body + 128, 64);\n    memcpy(t + 128 * N + 16 * i, body + 192, 16);")],
    "q6k_d_plane_index_both": [
        ("*d = rd16(t + 208 * N + 2 * i);", "*d = rd16(t + 208 * N + 2 * (N - 1 - i));"),
        ("wr16(t + 208 * N + 2 * i, d);", "wr16(t + 208 * N + 2 * (N - 1 - i), d);")],
    "q6k_high_plane_index_both": [
        ("memcpy(body + 128, t + 128 * N + 64 * i, 64);", "memcpy(body + 128, t + 128 * N + 64 * (N - 1 - i), 64);"),
        ("memcpy(t + 128 * N + 64 * i, body + 128, 64);", "memcpy(t + 128 * N + 64 * (N - 1 - i), body + 128, 64);")],
    "q6k_d_before_scales": [
        ("memcpy(body + 192, t + 192 * N + 16 * i, 16);\n    *d = rd16(t + 208 * N + 2 * i);",
         "memcpy(body + 192, t + 194 * N + 16 * i, 16);\n    *d = rd16(t + 192 * N + 2 * i);"),
        ("memcpy(t + 192 * N + 16 * i, body + 192, 16);\n    wr16(t + 208 * N + 2 * i, d);",
         "memcpy(t + 194 * N + 16 * i, body + 192, 16);\n    wr16(t + 192 * N + 2 * i, d);")],
    "bound_drops_min": (
        "double wh = d * sc * q4k_q(blk, 32 * j + i) - dmin * m;",
        "double wh = d * sc * q4k_q(blk, 32 * j + i);"),
}

RUNNER = r"""
import json, sys
sys.path[:0] = [{root!r}, {tests!r}]
import numpy as np
import oracle, oracle_pins as pins
lib = oracle.load({so!r})
rng = np.random.default_rng(1)
w = (rng.standard_normal((6, 512)) * 0.02).astype(np.float32)
w2 = (rng.standard_normal((6, 512)) * 0.002).astype(np.float32)
w3 = rng.standard_normal((6, 512)).astype(np.float32)
x = rng.standard_normal((2, 512)).astype(np.float32)
checks = {{
    "fp16": lambda: pins.check_fp16(lib),
    "layout_goldens": lambda: pins.check_layout_goldens(lib),
    "layout_probes": lambda: pins.check_layout_probes(lib),
    "act_cases": lambda: pins.check_act_cases(lib),
    "act_bounds": lambda: pins.check_act_bounds(lib),
    "act_overflow": lambda: pins.check_act_overflowing_inverse(lib),
    "q4k_quantizer": lambda: (pins.check_q4k_quantizer(lib, w), pins.check_q4k_quantizer(lib, w3),
                              pins.check_q4k_quantizer(lib, w2)),
    "q6k_quantizer": lambda: (pins.check_q6k_quantizer(lib, w), pins.check_q6k_quantizer(lib, w3),
                              pins.check_q6k_quantizer(lib, w2, True)),
    "bf_q4k": lambda: pins.check_gemv_bruteforce(lib, "q4k", w, x),
    "bf_q6k": lambda: pins.check_gemv_bruteforce(lib, "q6k", w, x),
    "onehot_q4k": lambda: pins.check_gemv_onehot(lib, "q4k", w),
    "onehot_q6k": lambda: pins.check_gemv_onehot(lib, "q6k", w),
    "special": lambda: pins.check_gemv_special(lib),
    "extremes": lambda: pins.check_gemv_extremes(lib),
    "q32_layout": lambda: pins.check_q32_layout_goldens(lib),
    "qk_tensors": lambda: pins.check_qk_tensor_goldens(lib),
    "q40_quantizer": lambda: (pins.check_q40_quantizer(lib, w), pins.check_q40_quantizer(lib, w3)),
    "q80_quantizer": lambda: (pins.check_q80_quantizer(lib, w), pins.check_q80_quantizer(lib, w3)),
    "q80_act_cases": lambda: [np.testing.assert_array_equal(
        oracle.q80_codes(oracle.quantize_q80(xc[None, :], lib=lib), 1, xc.size).reshape(-1), qc)
        for xc, qc, _ in pins.read_act_cases()],
    "bf_q40": lambda: pins.check_gemv_bruteforce(lib, "q40", w, x),
    "bf_q80": lambda: pins.check_gemv_bruteforce(lib, "q80", w, x),
    "onehot_q40": lambda: pins.check_gemv_onehot(lib, "q40", w),
    "onehot_q80": lambda: pins.check_gemv_onehot(lib, "q80", w),
}}
failed = []
for name, fn in checks.items():
    try:
        fn()
    except AssertionError:
        failed.append(name)
print(json.dumps(failed))
"""


def _run(tmp_path, name, source):
    src = tmp_path / (name + ".c")
    src.write_text(source)
    so = str(tmp_path / (name + ".so"))
    oracle.build(out=so, src=str(src))
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = RUNNER.format(root=root, tests=os.path.join(root, "tests"), so=so)
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    if proc.returncode != 0:
        # a mutant that aborts (int32 range check, bad code) has been caught as well
        return ["<crashed: %d>" % proc.returncode]
    return json.loads(proc.stdout.strip().splitlines()[-1])


def test_unmutated_oracle_passes_every_pin(tmp_path):
    with open(SRC) as f:
        assert _run(tmp_path, "control", f.read()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    with open(SRC) as f:
        text = f.read()
    edits = MUTANTS[name]
    for old, new in (edits if isinstance(edits, list) else [edits]):
        assert text.count(old) == 1, "mutation anchor not found once: %s" % name
        text = text.replace(old, new)
    failed = _run(tmp_path, name, text)
    assert failed, "no pin caught mutant %s" % name
