"""The host library's validation and planning under AddressSanitizer and
UndefinedBehaviorSanitizer: pa_api.cpp built with the host compiler's
sanitizers against stub launchers (tests/host_sanitizers/launch_stubs.cpp),
driven by a seeded fuzz of descriptors, options and CU counts through every
entry point (tests/host_sanitizers/plan_fuzz.cpp).  CPU only: no descriptor
address is dereferenced, and nothing reaches a kernel launcher."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitizers")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_host_library_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path / "plan_fuzz")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "paged_kv_cache_unified_amd", "csrc"),
           os.path.join(HERE, "plan_fuzz.cpp"), os.path.join(HERE, "launch_stubs.cpp"),
           os.path.join(ROOT, "paged_kv_cache_unified_amd", "csrc", "pa_api.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               HIP_VISIBLE_DEVICES="-1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert "ok" in r.stdout and "FAIL" not in r.stdout, r.stdout[-4000:]
