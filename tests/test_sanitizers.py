"""AddressSanitizer and UBSan builds of the CPU code, run without a GPU: the oracle
(oracle/oracle.c, driven through every entry point by tests/sanitize/oracle_driver.c)
and the library's host code (host.cpp: argument checks, the plan builder, status and
error texts, driven by tests/sanitize/host_driver.cpp with the device side replaced by
tests/sanitize/host_stubs.cpp).  Any sanitizer report fails the run (no recovery)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _build(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and ("asan" in r.stderr.lower() or "ubsan" in r.stderr.lower()):
        pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr[-3000:]


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _build(["gcc", "-std=c99", *SAN, "-I", os.path.join(ROOT, "oracle"),
            os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"),
            "-lm", "-o", exe])
    assert "harness done" in _run(exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_san")
    csrc = os.path.join(ROOT, "microscaling_fp4_attention_amd", "csrc")
    _build(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
            "-I", os.path.join(ROOT, "include"), "-I", csrc,
            os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"),
            os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"), os.path.join(csrc, "host.cpp"), "-o", exe])
    assert "harness done" in _run(exe)
