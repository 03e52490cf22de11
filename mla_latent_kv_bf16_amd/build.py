"""Build libmla_decode.so in-tree: hipcc for gfx950, one object per source,
compiled in parallel, then linked into a shared library next to this file."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmla_decode.so")
PROBE_LIB = os.path.join(HERE, "libmla_hbm_probe.so")  # measurement helper, not the decode

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          # packed fp32 instructions are kept out of every kernel
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # MFMA accumulators in VGPRs: with AGPR accumulators the register
          # allocator copies all 128 P.V accumulators into VGPRs on every
          # tile (for the rare rescale), and the kernels need ~130 more
          # registers in all
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          # only the C ABI (MLA_API in include/mla_decode.h) is exported
          "-fvisibility=hidden",
          "-I", os.path.join(ROOT, "include"), "-Wall"]
SOURCES = ["plan.cpp", "api.cpp", "quant.hip", "merge.hip", "stage1_fp8.hip", "stage1_mxfp4.hip",
           "stage1_fp8_rows.hip", "stage1_bf16.hip", "noalloc.hip"]
PROBE_SOURCES = ["hbm_probe.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str):
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(PROBE_SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
