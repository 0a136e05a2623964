"""The host side of the C ABI under the address and undefined-behaviour sanitizers.

mla_api.cpp (the planner, the table check and every argument check) is built
with g++ -fsanitize=address,undefined together with tests/host/hip_stubs.cpp
(stand-ins for the kernel launchers, which check every plan they are handed)
and tests/host/api_driver.cpp (600 random descriptions and lengths up to
400k, plus invalid calls), and run on the CPU.  Any out-of-bounds access,
use of freed memory, signed overflow or other undefined operation aborts the
run; so does a plan whose units do not cover each request exactly once.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_latent_kv_absorbed_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_planner_and_argument_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(CSRC, "mla_api.cpp"), os.path.join(HOST, "hip_stubs.cpp"),
           os.path.join(HOST, "api_driver.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), \
        (run.stdout[-2000:] + run.stderr[-4000:])
