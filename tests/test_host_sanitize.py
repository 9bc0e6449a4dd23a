"""Host C++ of the library under AddressSanitizer and UndefinedBehaviorSanitizer.

The parts of the library that run on the CPU and touch no GPU -- the weight
repacking into the device image (bf16 rounding, E4M3 codes with per-row
exponents, the head-major Q|K|V copy), the E4M3 and bf16 encoders, the
workspace plan and the aliasing test -- live in csrc/host.hpp, which is plain
C++.  tests/host/host_checks.cpp includes it and checks each part against a
definition written there independently; here it is built with g++ and both
sanitizers (no HIP compiler involved) and run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_code_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "host_checks"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "albert_transformer_amd", "csrc"),
           os.path.join(ROOT, "tests", "host", "host_checks.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "0 failures" in r.stdout
