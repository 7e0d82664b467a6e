"""The library's host half (layout construction, estimates, block tables,
meta blob, argument validation and marshalling of every C entry point)
built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and
driven through the C ABI by tests/host_asan/driver.cpp.  The kernel
launchers are replaced by counting stand-ins (tests/host_asan/
kernel_stubs.cpp), so no device is needed; the sanitizers abort on the first
report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "head_windowed_kv_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_asan")
ROCM_INCLUDE = "/opt/rocm/include"


def test_host_abi_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path / "hwkv_host_asan")
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "layout.cpp"), os.path.join(CSRC, "api.cpp"),
           os.path.join(HERE, "kernel_stubs.cpp"), os.path.join(HERE, "driver.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    if build.returncode != 0 and "asan" in build.stderr.lower():
        pytest.skip("sanitizer runtime not available: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "ok" in run.stdout
