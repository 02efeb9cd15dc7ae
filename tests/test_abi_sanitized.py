"""The C-ABI layer (fa_api.cpp: argument validation and dispatch) built with
the address and undefined-behaviour sanitizers, on the host only.

fa_api.cpp is compiled with g++ together with host stand-ins for the kernel
launchers (tests/abi_host/stub_launch.cpp, which record their arguments and
touch no device) and a driver (tests/abi_host/driver.cpp) that calls every
entry point with invalid arguments (each must be rejected with its status
before any launch), with valid ones up to the largest accepted sizes (each
must reach the launchers with the documented arguments), and with enum values
outside the named ones.  Any out-of-bounds access, leak, signed overflow or
invalid enum load stops the run.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "io_aware_exact_09_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "abi_host")


@pytest.fixture(scope="module")
def sanitized_driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path_factory.mktemp("abi_san") / "abi_driver")
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(CSRC, "fa_api.cpp"), os.path.join(HOST, "stub_launch.cpp"),
           os.path.join(HOST, "driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_abi_validation_under_sanitizers(sanitized_driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sanitized_driver], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out
    assert out.strip().startswith("ok "), out
