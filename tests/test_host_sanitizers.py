"""The library's host C++ under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): the randomized SVD of the weight split (关键设计 4), every argument
check, and the workspace layout planning over many geometries, compiled with
g++ from csrc/api.cpp and csrc/svd.cpp with the device launchers stubbed
(tests/host/sanitize_driver.cpp)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "w4a4_quantized_linear_cube_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"), reason="needs g++ and ROCm headers")
def test_host_code_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "sanitize_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(ROOT, "tests", "host", "sanitize_driver.cpp"), os.path.join(CSRC, "api.cpp"),
           os.path.join(CSRC, "svd.cpp"), "-o", exe, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-lpthread"]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "0 failures" in out, out[-2000:]
