"""The library's host code (size queries, launch heuristics, argument validation) built with
AddressSanitizer and UndefinedBehaviorSanitizer on the host side only and driven by
tests/host_sanitize_driver.cpp.  CPU only: no kernel is launched and no GPU is needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_mixture_experts_align_amd", "csrc")
# the sources whose host code the driver calls (the GEMM sources are covered through ctypes)
SOURCES = ["moe_api.hip", "moe_requant.hip", "moe_prepare.hip"]


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "host_sanitize_driver")
    cmd = [hipcc, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES],
           os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout[-4000:], r.stderr[-4000:])
