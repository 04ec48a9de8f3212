"""The host code that handles caller-supplied sizes and pointers, built with
AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU).

tests/sanitize_check.cpp links the oracle (oracle/oracle.c) and the C ABI's
argument validation (exact_io_aware_44_amd/csrc/fa_api.cpp, with the kernel
launchers replaced by counters) into one sanitized executable.  It calls every
entry point with invalid and extreme sizes (INT_MAX, INT_MIN, SIZE_MAX) and
with valid ones, and every oracle function on small inputs with results fixed
by the mathematics.  Any sanitizer report (out-of-bounds access, leak, signed
overflow, misaligned or null access) ends it with a non-zero status.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_44_amd", "csrc")
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]
CXX = ["-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
       "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr)
    return r


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None
                    or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"),
                    reason="needs gcc, g++ and the HIP headers")
def test_oracle_and_abi_validation_under_asan_ubsan(tmp_path):
    d = str(tmp_path)
    _run(["gcc", *SAN, "-std=c11", "-fopenmp", "-c", os.path.join(ROOT, "oracle", "oracle.c"),
          "-o", os.path.join(d, "oracle.o")])
    _run(["g++", *SAN, *CXX, "-c", os.path.join(CSRC, "fa_api.cpp"),
          "-o", os.path.join(d, "fa_api.o")])
    _run(["g++", *SAN, *CXX, "-c", os.path.join(ROOT, "tests", "sanitize_check.cpp"),
          "-o", os.path.join(d, "check.o")])
    exe = os.path.join(d, "sanitize_check")
    _run(["g++", *SAN, "-fopenmp", os.path.join(d, "check.o"), os.path.join(d, "fa_api.o"),
          os.path.join(d, "oracle.o"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="4")
    r = _run([exe], env=env, timeout=120)
    assert "sanitize ok" in r.stdout, r.stdout + r.stderr
