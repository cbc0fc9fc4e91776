"""Builds libqmoe.so (gfx950) in the package directory with hipcc."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqmoe.so")
SOURCES = ["api.cpp", "route.hip", "permute.hip", "gemm_bf16.hip", "gemm_bf16_tiled.hip", "gemm_prefill.hip", "gemm_prefill_rows.hip", "gemm_prefill_blk.hip", "gemm_prefill_blk_tiled.hip", "gemm_f32.hip", "combine.hip", "pack.hip", "quant.hip", "noalloc.hip", "gemm_prefill_sw.hip", "gemm_prefill_sw8.hip", "gemm_prefill_i8.hip", "rowsum.hip", "f16prep.hip", "gemm_prefill_h16.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
         # no packed fp32 instructions in generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # MFMA accumulators in ordinary VGPRs: the epilogues read them every scale block
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-I", os.path.join(HERE, "..", "include")]


# the 128-row per-row-scale kernel is built without that option: at two waves per SIMD it
# has 256 registers a wave and keeps its accumulators in VGPRs either way (both forms give
# the same code size and scratch; its shapes were measured in the default form)
NO_VGPR_FORM = {"gemm_prefill_rows.hip"}


def _flags(src: str):
    if src in NO_VGPR_FORM:
        out = list(FLAGS)
        i = out.index("-amdgpu-mfma-vgpr-form")
        del out[i - 1:i + 1]
        return out
    return FLAGS


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *_flags(src), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if r.stderr.strip():
        warn = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if warn:
            sys.stderr.write("\n".join(warn) + "\n")
    return obj


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
