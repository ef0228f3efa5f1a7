"""CPU: the C-ABI host layer (flashbev_api.cpp: argument validation, size arithmetic,
error text) built with AddressSanitizer and UndefinedBehaviorSanitizer against
host-only launcher stand-ins, and driven through every entry point with valid,
invalid and extreme arguments (tests/sanitize/harness.cpp).  Nothing touches a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_layer_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "fbev_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "camera_bev_view_amd", "csrc", "flashbev_api.cpp"),
           os.path.join(SAN, "launch_stubs.cpp"), os.path.join(SAN, "harness.cpp"), "-o", exe, "-lpthread"]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stdout[-4000:] + res.stderr[-4000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-4000:]
