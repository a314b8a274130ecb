"""Build libmoe_w4a16.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m quantized_mixture_experts_align_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_w4a16.so")
SOURCES = ["moe_api.hip", "moe_align.hip", "moe_prepare.hip", "moe_gemm.hip", "moe_gemm_int4.hip",
           "moe_gemm_nvfp4.hip", "moe_gemm_mxfp4.hip", "moe_gemm_int4zp.hip", "moe_gemm_stream_int4.hip",
           "moe_gemm_stream_nvfp4.hip", "moe_gemm_stream_mxfp4.hip", "moe_gemm_stream_int4zp.hip",
           "moe_gemm_int4zpf.hip", "moe_gemm_stream_int4zpf.hip",
           "moe_act_combine.hip", "moe_requant.hip"]
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions (v_pk_*_f32) are generated for device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: otherwise the loop-carried accumulators are copied
    # into AGPRs before every MFMA
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(jobs: int = 0, verbose: bool = False) -> str:
    """Compile every source and link the shared library; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    r = subprocess.run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    a = ap.parse_args()
    build(a.jobs, verbose=True)
    sys.exit(0)
