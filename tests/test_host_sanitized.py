"""The library's host arithmetic (plan tables and launch geometry, csrc/rd_host.cpp) built by the
host compiler with AddressSanitizer and UndefinedBehaviorSanitizer and checked against
independent computations (tests/host/host_checks.cpp): no GPU is needed, and any out-of-bounds
access, leak or undefined operation in table construction fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "range_doppler_focusing_amd", "csrc")


def test_host_tables_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "host_checks")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-Wall", "-Wextra", "-Werror", "-I", CSRC,
           os.path.join(ROOT, "tests", "host", "host_checks.cpp"), os.path.join(CSRC, "rd_host.cpp"),
           "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "host checks passed" in r.stdout
