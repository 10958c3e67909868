"""The C-ABI layer built for the host with AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

kvc_api.cpp is compiled with g++ next to launcher stubs that abort and a driver
that sends every entry point invalid arguments and workspace-size queries; the
driver must report every check passed with no sanitizer finding.  No GPU code is
built or run.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "kv_cache_compression_window_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_abi_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", "/opt/rocm/include", os.path.join(CSRC, "kvc_api.cpp"), os.path.join(HERE, "stub_launch.cpp"),
           os.path.join(HERE, "abi_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "all checks passed" in r.stdout, r.stdout + r.stderr
