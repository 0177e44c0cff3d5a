"""The matrix-core kernel issues its direct-to-LDS copies from inline assembly that sets M0 (the
LDS base of the copy) and names M0 as clobbered. The compiler may keep its own values in M0, so
this checks, in the gfx950 assembly of the library's own source, that M0 is only ever written
right before such a copy and read by nothing else. CPU only (hipcc cross-compiles); skipped
when hipcc is not there."""

import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_quantized_weight_act_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                    reason="hipcc not available")
def test_m0_only_feeds_the_lds_copies():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "qgemv_build", os.path.join(ROOT, "block_quantized_weight_act_amd", "build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "gemm_mfma.s")
        cmd = [HIPCC, *build.FLAGS, *build.FILE_FLAGS.get("gemm_mfma.hip", []), "-x", "hip",
               "-S", "--offload-device-only", os.path.join(CSRC, "gemm_mfma.hip"), "-o", out]
        subprocess.run(cmd, check=True, capture_output=True)
        lines = [ln.split(";")[0].strip() for ln in open(out)]
    insts = [ln for ln in lines if ln and not ln.startswith(".") and not ln.endswith(":")]
    copies = 0
    for i, ln in enumerate(insts):
        if not re.search(r"\bm0\b", ln):
            continue
        assert ln.startswith("s_mov_b32 m0,"), "M0 used outside the LDS copies: " + ln
        assert insts[i + 1].startswith("global_load_lds_dwordx4"), insts[i + 1]
        copies += 1
    assert copies > 0
