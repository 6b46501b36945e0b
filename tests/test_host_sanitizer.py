"""The C-ABI layer (api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

api.cpp is plain C++: it is built here with g++ and both sanitizers, linked
against host_sanitizer_stubs.cpp in place of the HIP kernels, and the argument
validation matrix of test_abi.py runs against that library in a child Python
(the sanitizer runtime preloaded, leak checking off for the interpreter's own
allocations). Any sanitizer report aborts the child. The stubs count every
call that reaches a launcher or device check, and test_abi.py asserts that no
call reaches one: every rejected or empty call returns before the GPU side. The
matrix runs twice, the second time with the device contract check (VFA_DEBUG)
switched on.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "varlen_flash_attention_amd", "csrc")


def _build(out_dir):
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, "libvfa_host_sanitized.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "api.cpp"), os.path.join(ROOT, "tests", "host_sanitizer_stubs.cpp"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    return out


@pytest.mark.parametrize("debug", ["0", "1"])
def test_abi_validation_under_sanitizers(debug):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    lib = _build(os.path.join(ROOT, "_build", "host_sanitizer"))
    asan = subprocess.check_output(["g++", "-print-file-name=libasan.so"], text=True).strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("the AddressSanitizer runtime is not installed")
    env = dict(os.environ, LD_PRELOAD=asan, VFA_TEST_LIBRARY=lib, VFA_DEBUG=debug,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"), "-k", "not exports"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    report = (r.stdout[-3000:] + "\n" + r.stderr[-3000:]).strip()
    assert r.returncode == 0, report
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, report
    assert " passed" in r.stdout, report
