"""Build libqgemv.so for gfx950 with hipcc, in-tree (block_quantized_weight_act_amd/_lib/).

Every source is compiled on each call (one hipcc process per file, in parallel), then linked
into one shared library. Flags:
  -ffp-contract=off     no implicit fused multiply-adds: the activation and weight quantizers
                        must round each float32 operation exactly as written, and the GEMV's
                        scale products must be rounded separately (the kernels use explicit
                        fmaf where a fused multiply-add is wanted)
  -packed-fp32-ops off  no v_pk_*_f32 instructions generated from float code
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(HERE, "_lib", "obj")
LIB = os.path.join(HERE, "_lib", "libqgemv.so")

SOURCES = ["gemv_multi.hip", "gemv_q4k.hip", "gemv_q6k.hip", "gemv_q40.hip", "gemv_q80.hip",
           "api.cpp", "graph.cpp", "gemm_mfma.hip", "gemm_i8.hip", "act_quant.hip", "reduce.hip", "weight_quant.hip", "read_probe.hip",
           "scratch.hip", "gemm_q32.hip", "gemm_q6k_mc.hip", "gemm_q32_i8.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


# Per-file additions. gemm_mfma.hip, gemm_i8.hip: matrix-core results in ordinary VGPRs, so the float
# work that reads them needs no accumulator-register copies (v_accvgpr_read) first.
FILE_FLAGS = {"gemm_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "gemm_i8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "gemm_q32.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "gemm_q6k_mc.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "gemm_q32_i8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError("hipcc failed on %s" % src)
    return obj


def build(jobs: int | None = None) -> str:
    """Compile all sources and link libqgemv.so. Returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError("link of libqgemv.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
