"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only; GPU-side sanitizers are not used).

``tests/host_sanitize/host_driver.cpp`` is compiled with
``split_kv_long_amd/csrc/fd_host.cpp`` (argument checks, planner, kernel
argument marshalling) against stub launchers that check what each kernel
would receive. It drives every entry point over 20000 seeded random shapes
(valid and invalid) with fake device addresses; any out-of-bounds access,
signed overflow or other undefined behaviour aborts the run.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = str(tmp_path / "host_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "split_kv_long_amd", "csrc"),
           "-isystem", os.path.join(rocm, "include"),
           os.path.join(ROOT, "split_kv_long_amd", "csrc", "fd_host.cpp"),
           os.path.join(ROOT, "tests", "host_sanitize", "host_driver.cpp"),
           "-o", exe]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                       env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.startswith("ok "), r.stdout
    launches = int(r.stdout.split()[1])
    assert launches > 1000        # the valid calls reached the launchers
