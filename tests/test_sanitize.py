"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU):
the CPU reference (oracle/nosa_oracle.c) run on small ragged inputs and bad
arguments, and the C ABI's host side (nosa_api.cpp: argument checks,
planning, workspace sizes) with its kernel launchers stubbed out.  Both are
built with gcc / g++ on lines of their own (no device code is compiled)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
ENV = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(build, exe):
    r = subprocess.run(build, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    return report


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    cmd = ["gcc", "-std=c99", *SAN, "-fopenmp", "-I", os.path.join(ROOT, "oracle"),
           os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "nosa_oracle.c"),
           "-lm", "-o", exe]
    assert "oracle driver: ok" in _run(cmd, exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not found")
def test_api_host_side_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_san")
    csrc = os.path.join(ROOT, "block_sparse_attention_nosa_amd", "csrc")
    cmd = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", csrc, os.path.join(HERE, "api_driver.cpp"),
           os.path.join(csrc, "nosa_api.cpp"), "-o", exe]
    assert "api driver: ok" in _run(cmd, exe)
