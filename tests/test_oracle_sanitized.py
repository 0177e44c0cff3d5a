"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, host code only)
runs every oracle pin without a report: no out-of-bounds access, use of freed memory, signed
overflow, misaligned access or shift past the width anywhere in the C code the pins reach
(the layouts, quantizers, integer GEMV, brute force, bound and fp16 codec)."""

import os
import subprocess
import sys

import pytest

import oracle
from test_oracle_mutants import RUNNER

SAN_FLAGS = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]


def _runtime(name):
    out = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's AddressSanitizer runtime is not installed")
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    so = str(tmp_path / "liboracle_san.so")
    oracle.build(out=so, extra_flags=SAN_FLAGS)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = RUNNER.format(root=root, tests=os.path.join(root, "tests"), so=so)
    env = dict(os.environ)
    # the interpreter is not instrumented: the ASan runtime must come first in the process
    env["LD_PRELOAD"] = _runtime("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          timeout=600, env=env)
    report = proc.stderr[-4000:]
    assert proc.returncode == 0, report
    assert "runtime error" not in proc.stderr and "AddressSanitizer" not in proc.stderr, report
    assert proc.stdout.strip().splitlines()[-1] == "[]", proc.stdout


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's AddressSanitizer runtime is not installed")
def test_sanitized_build_reports_a_planted_overflow(tmp_path):
    """Control: a copy of the oracle whose Q4_K header read runs 8 bytes past the last block is
    reported by the same build and run (so the clean run above means something)."""
    src = open(oracle._SRC).read()
    anchor = "memcpy(img, t + 128 * N + 16 * i, 16);"
    assert src.count(anchor) == 1
    bad = tmp_path / "oracle_overflow.c"
    bad.write_text(src.replace(anchor, "memcpy(img, t + 128 * N + 16 * i + 8, 16);"))
    so = str(tmp_path / "liboracle_overflow.so")
    oracle.build(out=so, src=str(bad), extra_flags=SAN_FLAGS)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = RUNNER.format(root=root, tests=os.path.join(root, "tests"), so=so)
    env = dict(os.environ, LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          timeout=600, env=env)
    assert proc.returncode != 0
    assert "heap-buffer-overflow" in proc.stderr
