"""The C ABI's host code (validation, aliasing rules, workspace plans) built
on its own with g++ under the address and undefined-behaviour sanitizers and
driven through every entry point (tests/sanitize/abi_checks.cpp), with the
device launchers replaced by stand-ins that only record that they were
reached.  CPU only; skipped where g++ or its sanitizer runtimes are missing."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "kalman_delta_rule_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_abi_host_code_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path / "abi_checks")
    sources = [os.path.join(CSRC, "kdn_api.cpp"), os.path.join(CSRC, "kdn_plan.cpp"),
               os.path.join(HERE, "sanitize", "launch_stubs.cpp"),
               os.path.join(HERE, "sanitize", "abi_checks.cpp")]
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    res = subprocess.run([gxx] + flags + sources + ["-o", exe], capture_output=True, text=True)
    if res.returncode != 0 and "asan" in res.stderr.lower():
        pytest.skip("sanitizer runtime not available: " + res.stderr[-300:])
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(run.stdout[-2000:], run.stderr[-2000:])
    assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-3000:]
    assert "all checks passed" in run.stdout
