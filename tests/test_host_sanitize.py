"""The host side of libdeltalog under AddressSanitizer and UndefinedBehavior-
Sanitizer, on the CPU: dl_api.hip (plain host code) is built with g++ and the
sanitizers, its kernel launchers replaced by recording stubs
(tests/host_sanitize.cpp), and driven through argument validation, overlap
checks, the lockstep, two-stage, no-alloc and per-slot schedules (every
recorded launch checked against the documented schedule) and a thousand
handle life cycles, with leak detection on."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_host_api_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Werror",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "recurrent_state_update_amd", "csrc"),
           "-x", "c++", os.path.join(HERE, "host_sanitize.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report
    assert "ERROR:" not in report and "runtime error" not in report, report
    assert "host API checks passed" in r.stdout
