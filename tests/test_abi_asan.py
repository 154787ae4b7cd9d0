"""The C ABI's host-side checks under AddressSanitizer and UBSan (CPU only).

moe_abi.cpp is compiled with g++ and the sanitizers, linked against host-only
stand-ins of the kernel launchers (tests/asan/launch_stubs.cpp) and run by a
driver (tests/asan/abi_driver.cpp) that walks every entry point through its
accepted and rejected arguments: each case must return its status and reach a
launcher only when the arguments are accepted, with no sanitizer report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_abi_checks_under_address_sanitizer(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path / "abi_asan")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "dropless_mixture_experts_amd", "csrc"),
           os.path.join(ROOT, "dropless_mixture_experts_amd", "csrc", "moe_abi.cpp"),
           os.path.join(ROOT, "tests", "asan", "launch_stubs.cpp"),
           os.path.join(ROOT, "tests", "asan", "abi_driver.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=60)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert r.stdout.startswith("ok ") and "ERROR: AddressSanitizer" not in r.stderr
