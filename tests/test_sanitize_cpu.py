"""The C ABI's host code (validation, planners, layout model: csrc/api.cpp and
csrc/layout.cpp) built with AddressSanitizer and UndefinedBehaviorSanitizer and driven
through every host path by tests/sanitize/driver.cpp; the kernel launchers are host-only
stand-ins (tests/sanitize/stub_kernels.cpp), so no GPU is needed.  Any sanitizer report
or wrong status fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_shared_expert_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")


def test_host_code_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path / "smlp_sanitize")
    srcs = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "layout.cpp"),
            os.path.join(SAN, "stub_kernels.cpp"), os.path.join(SAN, "driver.cpp")]
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", exe, "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib", "-pthread"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "all checks passed" in out
