"""Address and undefined-behaviour sanitizer builds of the host code (CPU only).

Two host programs are built with g++ -fsanitize=address,undefined and run:
  - the C-ABI validation layer (block_scaled_fp4_gemm_amd/csrc/api.cpp)
    against a host-only stand-in for the HIP runtime header, with the kernel
    launchers replaced by recorders (tests/sanitize/api_driver.cpp);
  - the plain C++ oracle (oracle/cpu_oracle.cpp) on small and edge-sized
    inputs (tests/sanitize/oracle_driver.cpp).
No GPU code is built here. Any sanitizer report fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-pthread"]

GXX = shutil.which("g++")
pytestmark = pytest.mark.skipif(GXX is None, reason="g++ not found")


def _build_and_run(tmp_path, name, sources, extra=()):
    exe = os.path.join(str(tmp_path), name)
    r = subprocess.run([GXX, *FLAGS, *extra, *sources, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    return r.stdout


def test_api_validation_under_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "api_san",
                         [os.path.join(ROOT, "block_scaled_fp4_gemm_amd", "csrc", "api.cpp"),
                          os.path.join(SAN, "api_driver.cpp")],
                         ["-I" + os.path.join(SAN, "hip_stub"), "-I" + os.path.join(ROOT, "include")])
    assert "api sanitizer driver: ok" in out


def test_cpu_oracle_under_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "oracle_san",
                         [os.path.join(ROOT, "oracle", "cpu_oracle.cpp"), os.path.join(SAN, "oracle_driver.cpp")],
                         ["-ffp-contract=off"])
    assert "oracle sanitizer driver: ok" in out
