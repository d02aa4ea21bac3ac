"""Host code under AddressSanitizer and UBSan (CPU only).

Two programs are built with the host compilers and run: the CPU oracle driven
on small inputs (tests/sanitize/oracle_driver.c), and the library's C-ABI
layer (qsa_api.cpp: every argument check, workspace layout and launch
decision) with its kernel launchers replaced by recording stand-ins
(tests/sanitize/host_stubs.cpp), driven through every entry point
(tests/sanitize/api_driver.cpp).  Any memory error or undefined behaviour
aborts the program, which fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "top_sparse_attention_amd", "csrc")
ROCM = "/opt/rocm"
SAN_FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer"]
# The HIP runtime's own allocations are not this code's; leaks are not checked.
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "oracle_driver"
    r = _run(["gcc", "-std=c11", *SAN_FLAGS, os.path.join(ROOT, "oracle", "qsa_oracle.c"),
              os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", str(exe)])
    assert r.returncode == 0, r.stderr
    r = _run([str(exe)], env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all oracle checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_host_api_under_sanitizers(tmp_path):
    hip = os.path.join(ROCM, "lib", "libamdhip64.so")
    if shutil.which("g++") is None or not os.path.exists(hip):
        pytest.skip("g++ or the HIP runtime library not available")
    exe = tmp_path / "api_driver"
    r = _run(["g++", "-std=c++17", *SAN_FLAGS, "-D__HIP_PLATFORM_AMD__",
              "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
              "-I", CSRC, "-I", SAN, os.path.join(CSRC, "qsa_api.cpp"),
              os.path.join(SAN, "host_stubs.cpp"), os.path.join(SAN, "api_driver.cpp"),
              "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
              "-o", str(exe)])
    assert r.returncode == 0, r.stderr
    r = _run([str(exe)], env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all host checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
