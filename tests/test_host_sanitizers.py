"""The host runtime's argument validation under AddressSanitizer and UndefinedBehaviorSanitizer.

td_api.cpp is compiled for the host with g++ -fsanitize=address,undefined (the kernel
launchers replaced by host stand-ins, tests/host_check/stubs.cpp) and linked with
tests/host_check/abi_host_check.cpp, which calls every entry point with invalid arguments.
Any out-of-bounds access, leak in the library's own code, or undefined behaviour on those
paths aborts the run.  CPU only; skipped where g++ or the HIP runtime library is missing.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def test_abi_validation_is_clean_under_asan_and_ubsan(tmp_path):
    if not shutil.which("g++") or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("needs g++ and the HIP runtime library")
    exe = tmp_path / "abi_host_check"
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           *SAN, os.path.join(ROOT, "block_diffusion_lm_step_amd", "csrc", "td_api.cpp"),
           os.path.join(ROOT, "tests", "host_check", "stubs.cpp"),
           os.path.join(ROOT, "tests", "host_check", "abi_host_check.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    supp = tmp_path / "lsan.supp"
    supp.write_text("leak:libamdhip64\nleak:libhsa-runtime64\nleak:librocprofiler\n")
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=1:detect_leaks=1:verify_asan_link_order=0",
               LSAN_OPTIONS=f"suppressions={supp}", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert " 0 failed" in r.stdout
